// C ABI of the overlap-save FIR library: plans, filter set-up, execution
// and state handling.  Argument meaning, ownership and error behaviour are
// documented in include/firols.h.
#include "firols.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <new>
#include <utility>
#include <vector>

#include "kernels.hpp"
#include "plan.hpp"

namespace {

using firols::launch_copy;

int ilog2_pow2(int64_t n) {
    if (n <= 0 || (n & (n - 1))) return -1;
    int l = 0;
    while ((int64_t(1) << l) < n) ++l;
    return l;
}

bool on_plan_device(const fir_ols_plan_s *p) {
    int d = -1;
    return hipGetDevice(&d) == hipSuccess && d == p->device;
}

void release(fir_ols_plan_s *p) {
    release_host_stream(p);
    (void)hipFree(p->tw_top);
    (void)hipFree(p->scratch);
    (void)hipFree(p->err);
    (void)hipFree(p->H);
    (void)hipFree(p->tw);
    (void)hipFree(p->taps);
    (void)hipFree(p->state[0]);
    (void)hipFree(p->state[1]);
    delete p;
}

int64_t state_len(const fir_ols_plan_s *p) { return p->nchan * (p->M - 1); }

bool is_multi(const fir_ols_plan_s *p) { return p->logn > firols::kSplitLogN; }
bool is_split(const fir_ols_plan_s *p) { return p->logn == firols::kSplitLogN; }
bool is_big(const fir_ols_plan_s *p) { return p->logn == firols::kBigLogN; }
bool is_mid(const fir_ols_plan_s *p) { return p->logn == firols::kMidLogN; }
// split and multi-pass paths: H in the split order
bool host_response(const fir_ols_plan_s *p) { return p->logn > firols::kBigLogN; }
// geometry id of the plan's table builders (fused and half-resident paths)
int table_geometry(const fir_ols_plan_s *p) {
    return is_big(p)   ? firols::big_geometry()
           : is_mid(p) ? firols::mid_geometry()
                       : firols::fused_geometry(p->logn);
}

int upload_freq_response(fir_ols_plan_t p, const float *H_host, hipStream_t s);

}  // namespace

extern "C" {

int fir_ols_plan(fir_ols_plan_t *out, int64_t M, int64_t N, int64_t nchan) {
    if (!out) return FIR_OLS_ERR_INVALID_ARG;
    *out = nullptr;
    const int logn = ilog2_pow2(N);
    if (logn < 0 || M < 1 || M > N || nchan < 1) return FIR_OLS_ERR_INVALID_ARG;
    if (logn < firols::kMinLogN || logn > firols::kMaxLogN) return FIR_OLS_ERR_UNSUPPORTED;
    if (nchan > (int64_t)1 << 30 || (M - 1) * nchan > ((int64_t)1 << 40))
        return FIR_OLS_ERR_UNSUPPORTED;

    fir_ols_plan_s *p = new (std::nothrow) fir_ols_plan_s;
    if (!p) return FIR_OLS_ERR_OOM;
    if (hipGetDevice(&p->device) != hipSuccess) {
        delete p;
        return FIR_OLS_ERR_HIP;
    }
    p->logn = logn;
    p->M = M;
    p->N = N;
    p->L = N - M + 1;
    p->nchan = nchan;
    const bool split = is_split(p), multi = is_multi(p);
    p->max_groups = multi       ? firols::multi_max_groups(p->device)
                    : split     ? firols::split_max_groups(p->device)
                    : is_big(p) ? firols::big_max_groups(p->device)
                    : is_mid(p) ? firols::mid_max_groups(p->device)
                                : firols::fused_max_groups(logn, p->device);
    (void)hipGetLastError();

    const int ntw = split || multi ? firols::split_sub_twiddle_count()
                                   : firols::twiddle_count(table_geometry(p));
    const int64_t ntop = multi   ? firols::multi_top_twiddle_count(logn)
                         : split ? firols::split_top_twiddle_count(logn)
                                 : 0;
    // split: the paired kernel's flags (one slot's worth), then one slot per
    // workgroup of the one-workgroup kernel
    const int64_t nscratch =
        multi   ? (int64_t)firols::multi_batch_units(logn) * N
        : split ? (int64_t)(p->max_groups + 1) * firols::split_slot_elems(logn)
                : 0;
    if (split) {
        p->pair_nq = firols::pair_queue_count(p->device);
        p->pair_lead = firols::pair_lead();
        p->pair_hold = firols::pair_hold_ready();
        p->pair_groups = firols::pair_max_groups(p->device);
        (void)hipGetLastError();
    }
    const size_t sbytes = (size_t)state_len(p) * sizeof(float2);
    bool ok = hipMalloc(&p->H, N * sizeof(float2)) == hipSuccess &&
              hipMalloc(&p->tw, (size_t)(ntw > 0 ? ntw : 1) * sizeof(float2)) == hipSuccess &&
              hipMalloc(&p->taps, N * sizeof(float2)) == hipSuccess &&
              hipMalloc(&p->err, sizeof(unsigned)) == hipSuccess &&
              hipMemset(p->err, 0, sizeof(unsigned)) == hipSuccess;
    if (ok && sbytes) {
        ok = hipMalloc(&p->state[0], sbytes) == hipSuccess &&
             hipMalloc(&p->state[1], sbytes) == hipSuccess;
    }
    if (ok && (split || multi)) {
        ok = hipMalloc(&p->tw_top, (size_t)ntop * sizeof(float2)) == hipSuccess &&
             hipMalloc(&p->scratch, (size_t)nscratch * sizeof(float2)) == hipSuccess;
        p->scratch_elems = nscratch;
    }
    if (!ok) {
        (void)hipGetLastError();
        release(p);
        return FIR_OLS_ERR_OOM;
    }

    std::vector<float2> tw((size_t)(ntw > 0 ? ntw : 1), make_float2(1.f, 0.f));
    std::vector<float2> top((size_t)(ntop > 0 ? ntop : 1));
    if (multi) {
        firols::build_twiddles(firols::big_geometry(), tw.data());
        firols::build_multi_top_twiddles(logn, top.data());
    } else if (split) {
        firols::build_split_twiddles(logn, tw.data(), top.data());
    } else {
        firols::build_twiddles(table_geometry(p), tw.data());
    }
    hipError_t e = hipMemcpy(p->tw, tw.data(), tw.size() * sizeof(float2), hipMemcpyHostToDevice);
    if (e == hipSuccess && (split || multi))
        e = hipMemcpy(p->tw_top, top.data(), (size_t)ntop * sizeof(float2), hipMemcpyHostToDevice);
    if (e == hipSuccess && sbytes) e = launch_copy(p->state[0], nullptr, state_len(p), nullptr);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        release(p);
        return FIR_OLS_ERR_HIP;
    }
    *out = p;
    return FIR_OLS_OK;
}


int fir_ols_set_taps(fir_ols_plan_t p, const float *h_host, int64_t M, int is_complex,
                     void *stream) {
    if (!p || !h_host || M != p->M) return FIR_OLS_ERR_INVALID_ARG;
    if (!on_plan_device(p)) return FIR_OLS_ERR_DEVICE;
    std::vector<float2> padded((size_t)p->N, make_float2(0.f, 0.f));
    for (int64_t m = 0; m < M; ++m)
        padded[m] = is_complex ? make_float2(h_host[2 * m], h_host[2 * m + 1])
                               : make_float2(h_host[m], 0.f);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipMemcpyAsync(p->taps, padded.data(), p->N * sizeof(float2),
                                  hipMemcpyHostToDevice, s);
    if (e == hipSuccess)
        e = host_response(p) ? firols::launch_split_plan_taps(p->logn, p->taps, p->H, p->tw, s)
            : is_big(p)      ? firols::launch_big_plan_taps(p->taps, p->H, p->tw, s)
            : is_mid(p)      ? firols::launch_mid_plan_taps(p->taps, p->H, p->tw, s)
                             : firols::launch_plan_taps(p->logn, p->taps, p->H, p->tw, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return FIR_OLS_ERR_HIP;
    p->has_filter = true;
    p->real_filter = !is_complex;
    return FIR_OLS_OK;
}

int fir_ols_set_freq_response(fir_ols_plan_t p, const float *H_host, int64_t N, void *stream) {
    if (!p || !H_host || N != p->N) return FIR_OLS_ERR_INVALID_ARG;
    if (!on_plan_device(p)) return FIR_OLS_ERR_DEVICE;
    const int st = upload_freq_response(p, H_host, (hipStream_t)stream);
    if (st == FIR_OLS_OK) p->real_filter = false;
    return st;
}

}  // extern "C"

namespace {

// H (unscaled, natural bin order, interleaved complex) scaled by 1/N into
// the kernels' order on the device.
int upload_freq_response(fir_ols_plan_t p, const float *H_host, hipStream_t s) {
    const int64_t N = p->N;
    std::vector<int64_t> perm((size_t)N);
    if (host_response(p))
        firols::build_split_h_permutation(p->logn, perm.data());
    else
        firols::build_h_permutation(table_geometry(p), perm.data());
    const float scale = 1.0f / (float)N;   // exact: N is a power of two
    std::vector<float2> Hk((size_t)N);
    for (int64_t i = 0; i < N; ++i) {
        const int64_t b = perm[i];
        Hk[i] = make_float2(H_host[2 * b] * scale, H_host[2 * b + 1] * scale);
    }
    hipError_t e = hipMemcpyAsync(p->H, Hk.data(), N * sizeof(float2), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return FIR_OLS_ERR_HIP;
    p->has_filter = true;
    return FIR_OLS_OK;
}

}  // namespace

namespace firols {

// fir_ols_execute (real == false: complex64 [nchan][stride]) and
// fir_ols_execute_real (real == true: float32 [2 nchan][stride]) on a
// given scratch area of scratch_elems float2 values, which the split
// (N = 65536) and multi-pass (N > 65536) kernels use: the split path runs at
// most one workgroup per N-sample slot of it, the multi-pass path moves the
// call's blocks through it in batches of as many blocks as it holds.
int execute_with_scratch(fir_ols_plan_s *p, const void *x_dev, void *y_dev, int64_t nsamples,
                         int64_t stride, void *stream, bool real, float2 *scratch,
                         int64_t scratch_elems) {
    if (!p || nsamples < 0) return FIR_OLS_ERR_INVALID_ARG;
    if (!p->has_filter) return FIR_OLS_ERR_NO_FILTER;
    if (real && !p->real_filter) return FIR_OLS_ERR_UNSUPPORTED;
    if (nsamples == 0) return FIR_OLS_OK;
    if (!x_dev || !y_dev || stride < nsamples) return FIR_OLS_ERR_INVALID_ARG;
    const uintptr_t align = real ? 3 : 7;
    if (((uintptr_t)x_dev | (uintptr_t)y_dev) & align) return FIR_OLS_ERR_ALIGN;
    const int64_t rows = real ? 2 * p->nchan : p->nchan;
    const int64_t item = real ? (int64_t)sizeof(float) : (int64_t)sizeof(float2);
    if (stride > ((int64_t)1 << 50) / rows) return FIR_OLS_ERR_INVALID_ARG;
    const int64_t span = ((rows - 1) * stride + nsamples) * item;
    const uintptr_t xa = (uintptr_t)x_dev, ya = (uintptr_t)y_dev;
    if (xa < ya + (uintptr_t)span && ya < xa + (uintptr_t)span) return FIR_OLS_ERR_ALIAS;
    if (!on_plan_device(p)) return FIR_OLS_ERR_DEVICE;

    const int64_t nblk = (nsamples + p->L - 1) / p->L;
    const hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipSuccess;
    if (is_multi(p)) {
        const int64_t batch = scratch_elems / p->N;
        if (!scratch || batch < 1) return FIR_OLS_ERR_UNSUPPORTED;
        MultiArgs a;
        a.x = (const float2 *)x_dev;
        a.y = (float2 *)y_dev;
        a.s0_old = p->state[p->parity];
        a.s0_new = p->state[p->parity ^ 1];
        a.H = p->H;
        a.tw = p->tw;
        a.tw_top = p->tw_top;
        a.scratch = scratch;
        a.nsamples = nsamples;
        a.stride = stride;
        a.nblk = nblk;
        a.u0 = 0;
        a.nu = 0;
        a.M = (int)p->M;
        a.L = (int)p->L;
        a.nchan = (int)p->nchan;
        e = launch_multi(p->logn, a, p->max_groups, batch, s, real);
    } else if (is_split(p)) {
        // the scratch starts with the paired kernel's flags (one slot's
        // worth), then one slot per workgroup of the one-workgroup kernel
        const int64_t slot = split_slot_elems(p->logn);
        const int64_t slots = scratch_elems / slot - 1;
        if (!scratch || slots < 1) return FIR_OLS_ERR_UNSUPPORTED;
        // blocks whose L outputs are all valid go to the paired kernel; a
        // partial last block to the one-workgroup kernel
        const int64_t nfull = nsamples / p->L;
        if (nfull > 0) {
            PairArgs a;
            a.x = (const float2 *)x_dev;
            a.y = (float2 *)y_dev;
            a.s0_old = p->state[p->parity];
            a.s0_new = p->state[p->parity ^ 1];
            a.H = p->H;
            a.tw = p->tw;
            a.tw_top = p->tw_top;
            a.sync = reinterpret_cast<unsigned *>(scratch);
            a.nsamples = nsamples;
            a.stride = stride;
            a.nblk = nblk;
            a.nfull = nfull;
            a.u0 = 0;
            a.nu = 0;
            a.nq = p->pair_nq;
            a.lead = p->pair_lead;
            a.hold_ready = p->pair_hold ? 1 : 0;
            a.err = p->err;
            a.wait_ticks = firols::pair_wait_ticks(p->pair_hold);
            a.M = (int)p->M;
            a.L = (int)p->L;
            a.nchan = (int)p->nchan;
            e = launch_pair(a, p->pair_groups, s, real);
        }
        if (e == hipSuccess && nfull < nblk) {
            const int groups = (int)(slots < p->max_groups ? slots : p->max_groups);
            SplitArgs a;
            a.x = (const float2 *)x_dev;
            a.y = (float2 *)y_dev;
            a.s0_old = p->state[p->parity];
            a.s0_new = p->state[p->parity ^ 1];
            a.H = p->H;
            a.tw = p->tw;
            a.tw_top = p->tw_top;
            a.scratch = scratch + slot;
            a.nsamples = nsamples;
            a.stride = stride;
            a.nblk = nblk;
            a.blk0 = nfull;
            a.M = (int)p->M;
            a.L = (int)p->L;
            a.nchan = (int)p->nchan;
            e = launch_split(p->logn, a, groups, s, real);
        }
    } else {
        FusedArgs a;
        a.x = (const float2 *)x_dev;
        a.y = (float2 *)y_dev;
        a.s0_old = p->state[p->parity];
        a.s0_new = p->state[p->parity ^ 1];
        a.H = p->H;
        a.tw = p->tw;
        a.nsamples = nsamples;
        a.stride = stride;
        a.nblk = nblk;
        a.M = (int)p->M;
        a.L = (int)p->L;
        a.nchan = (int)p->nchan;
        e = is_big(p)   ? launch_big(a, p->max_groups, s, real)
            : is_mid(p) ? launch_mid(a, p->max_groups, s, real)
                        : launch_fused(p->logn, a, p->max_groups, s, real);
    }
    if (e != hipSuccess) return FIR_OLS_ERR_HIP;
    if (p->M > 1) p->parity ^= 1;
    return FIR_OLS_OK;
}

}  // namespace firols

extern "C" {

int fir_ols_execute(fir_ols_plan_t p, const void *x_dev, void *y_dev, int64_t nsamples,
                    int64_t chan_stride, void *stream) {
    return firols::execute_with_scratch(p, x_dev, y_dev, nsamples, chan_stride, stream, false,
                                        p ? p->scratch : nullptr, p ? p->scratch_elems : 0);
}

int fir_ols_execute_real(fir_ols_plan_t p, const void *x_dev, void *y_dev, int64_t nsamples,
                         int64_t row_stride, void *stream) {
    return firols::execute_with_scratch(p, x_dev, y_dev, nsamples, row_stride, stream, true,
                                        p ? p->scratch : nullptr, p ? p->scratch_elems : 0);
}

int fir_ols_set_state(fir_ols_plan_t p, const void *s0_dev, void *stream) {
    if (!p) return FIR_OLS_ERR_INVALID_ARG;
    if (p->M == 1) return FIR_OLS_OK;
    if (s0_dev && ((uintptr_t)s0_dev & 7)) return FIR_OLS_ERR_ALIGN;
    if (!on_plan_device(p)) return FIR_OLS_ERR_DEVICE;
    hipError_t e = launch_copy(p->state[p->parity], (const float2 *)s0_dev, state_len(p),
                               (hipStream_t)stream);
    return e == hipSuccess ? FIR_OLS_OK : FIR_OLS_ERR_HIP;
}

int fir_ols_get_state(fir_ols_plan_t p, void *s0_out_dev, void *stream) {
    if (!p) return FIR_OLS_ERR_INVALID_ARG;
    if (p->M == 1) return FIR_OLS_OK;
    if (!s0_out_dev) return FIR_OLS_ERR_INVALID_ARG;
    if ((uintptr_t)s0_out_dev & 7) return FIR_OLS_ERR_ALIGN;
    if (!on_plan_device(p)) return FIR_OLS_ERR_DEVICE;
    hipError_t e = launch_copy((float2 *)s0_out_dev, p->state[p->parity], state_len(p),
                               (hipStream_t)stream);
    return e == hipSuccess ? FIR_OLS_OK : FIR_OLS_ERR_HIP;
}

int fir_ols_check(fir_ols_plan_t p, void *stream) {
    if (!p) return FIR_OLS_ERR_INVALID_ARG;
    if (!on_plan_device(p)) return FIR_OLS_ERR_DEVICE;
    if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return FIR_OLS_ERR_HIP;
    unsigned h = 0;
    if (hipMemcpy(&h, p->err, sizeof h, hipMemcpyDeviceToHost) != hipSuccess)
        return FIR_OLS_ERR_HIP;
    if (h == 0) return FIR_OLS_OK;
    const unsigned zero = 0;
    if (hipMemcpy(p->err, &zero, sizeof zero, hipMemcpyHostToDevice) != hipSuccess)
        return FIR_OLS_ERR_HIP;
    return FIR_OLS_ERR_TIMEOUT;
}

int fir_ols_destroy(fir_ols_plan_t p) {
    if (!p) return FIR_OLS_OK;
    const int dev = p->device;
    int old = -1;
    hipError_t e = hipGetDevice(&old);
    if (e == hipSuccess && old != dev) e = hipSetDevice(dev);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    release(p);
    if (old >= 0 && old != dev) (void)hipSetDevice(old);
    return e == hipSuccess ? FIR_OLS_OK : FIR_OLS_ERR_HIP;
}

int64_t fir_ols_choose_n(int64_t M) {
    // blocks per second of N = 2^8 .. 2^20 on MI355X, measured by
    // order_fir_filtering_amd/tune_n.py (one call of many blocks per N)
    static const double kBlocksPerSecond[] = {
        1413348091.7, 722691855.1, 394924269.1,
        174677774.3, 73970396.6, 21268569.2,
        15491336.9, 7209844.3, 2557594.1,
        765870.6, 376224.9, 191183.2,
        94173.3
    };
    if (M < 1) return FIR_OLS_ERR_INVALID_ARG;
    int64_t best = FIR_OLS_ERR_UNSUPPORTED;
    double best_rate = 0.0;
    for (int logn = 8; logn <= firols::kMaxLogN; ++logn) {
        const int64_t N = (int64_t)1 << logn;
        if (N < M) continue;
        const double rate = (double)(N - M + 1) * kBlocksPerSecond[logn - 8];
        if (rate > best_rate) {
            best_rate = rate;
            best = N;
        }
    }
    return best;
}

int64_t fir_ols_block_length(fir_ols_plan_t p) {
    return p ? p->L : (int64_t)FIR_OLS_ERR_INVALID_ARG;
}

const char *fir_ols_status_string(int status) {
    switch (status) {
        case FIR_OLS_OK: return "ok";
        case FIR_OLS_ERR_INVALID_ARG: return "invalid argument";
        case FIR_OLS_ERR_UNSUPPORTED: return "unsupported size";
        case FIR_OLS_ERR_NO_FILTER: return "no filter set";
        case FIR_OLS_ERR_ALIAS: return "input and output overlap";
        case FIR_OLS_ERR_ALIGN: return "pointer not aligned to its element size";
        case FIR_OLS_ERR_OOM: return "device allocation failed";
        case FIR_OLS_ERR_HIP: return "HIP runtime error";
        case FIR_OLS_ERR_DEVICE: return "current device is not the plan's device";
        case FIR_OLS_ERR_TIMEOUT: return "a kernel's wait for another workgroup ran out";
        default: return "unknown status";
    }
}

}  // extern "C"
