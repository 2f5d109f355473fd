// C ABI of the polyphase filter-bank channelizer: plans, taps, calls and
// state.  Argument meaning, ownership and error behaviour are documented
// in include/firpfb.h.
#include "firpfb.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <new>
#include <vector>

#include "kernels.hpp"
#include "pfb.hpp"

struct fir_pfb_plan_s {
    int device = 0;
    int K = 0, D = 0, Nh = 0, T = 0, TM = 0;
    float *taps = nullptr;        // T * K taps, zero past Nh
    float2 *tw = nullptr;         // K-point FFT twiddles
    float2 *phase = nullptr;      // exp(-2 pi j e / K), e < K
    float2 *state[2] = {nullptr, nullptr};   // Nh - 1 samples each
    int parity = 0;
    int64_t pos = 0;              // stream time of the next sample
    int max_groups = 0;
    bool has_taps = false;
};

namespace {

bool on_device(const fir_pfb_plan_s *p) {
    int d = -1;
    return hipGetDevice(&d) == hipSuccess && d == p->device;
}

void release(fir_pfb_plan_s *p) {
    (void)hipFree(p->taps);
    (void)hipFree(p->tw);
    (void)hipFree(p->phase);
    (void)hipFree(p->state[0]);
    (void)hipFree(p->state[1]);
    delete p;
}

}  // namespace

extern "C" {

int fir_pfb_plan(fir_pfb_plan_t *out, int64_t K, int64_t D, int64_t Nh) {
    if (!out) return FIR_OLS_ERR_INVALID_ARG;
    *out = nullptr;
    if (K < 1 || (K & (K - 1)) || D < 1 || D > K || K % D || Nh < 1)
        return FIR_OLS_ERR_INVALID_ARG;
    if (K < (1 << firpfb::kMinLogK) || K > (1 << firpfb::kMaxLogK) ||
        Nh > firpfb::kMaxTapsPerBranch * K)
        return FIR_OLS_ERR_UNSUPPORTED;
    const int T = firpfb::taps_per_branch((int)K, (int)Nh);
    const int TM = T ? firpfb::tile_outputs((int)K, (int)D, T) : 0;
    if (!T || !TM) return FIR_OLS_ERR_UNSUPPORTED;

    fir_pfb_plan_s *p = new (std::nothrow) fir_pfb_plan_s;
    if (!p) return FIR_OLS_ERR_OOM;
    if (hipGetDevice(&p->device) != hipSuccess) {
        delete p;
        return FIR_OLS_ERR_HIP;
    }
    p->K = (int)K;
    p->D = (int)D;
    p->Nh = (int)Nh;
    p->T = T;
    p->TM = TM;
    p->max_groups = firpfb::max_groups(p->K, T, p->device);
    (void)hipGetLastError();
    const int ntw = firpfb::twiddle_count(p->K);
    const size_t sbytes = (size_t)(Nh - 1) * sizeof(float2);
    bool ok = hipMalloc(&p->taps, (size_t)T * K * sizeof(float)) == hipSuccess &&
              hipMalloc(&p->tw, (size_t)(ntw > 0 ? ntw : 1) * sizeof(float2)) == hipSuccess &&
              hipMalloc(&p->phase, (size_t)K * sizeof(float2)) == hipSuccess;
    if (ok && sbytes)
        ok = hipMalloc(&p->state[0], sbytes) == hipSuccess &&
             hipMalloc(&p->state[1], sbytes) == hipSuccess;
    if (!ok) {
        (void)hipGetLastError();
        release(p);
        return FIR_OLS_ERR_OOM;
    }
    std::vector<float2> tw((size_t)(ntw > 0 ? ntw : 1), make_float2(1.f, 0.f));
    firpfb::build_twiddles(p->K, tw.data());
    std::vector<float2> ph((size_t)K);
    for (int64_t e = 0; e < K; ++e) {
        const double a = -2.0 * M_PI * (double)e / (double)K;
        ph[e] = make_float2((float)std::cos(a), (float)std::sin(a));
    }
    hipError_t e = hipMemcpy(p->tw, tw.data(), tw.size() * sizeof(float2), hipMemcpyHostToDevice);
    if (e == hipSuccess)
        e = hipMemcpy(p->phase, ph.data(), ph.size() * sizeof(float2), hipMemcpyHostToDevice);
    if (e == hipSuccess && sbytes)
        e = firols::launch_copy(p->state[0], nullptr, Nh - 1, nullptr);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        release(p);
        return FIR_OLS_ERR_HIP;
    }
    *out = p;
    return FIR_OLS_OK;
}

int fir_pfb_set_taps(fir_pfb_plan_t p, const float *h_host, int64_t Nh, void *stream) {
    if (!p || !h_host || Nh != p->Nh) return FIR_OLS_ERR_INVALID_ARG;
    if (!on_device(p)) return FIR_OLS_ERR_DEVICE;
    std::vector<float> t((size_t)p->T * p->K, 0.f);
    for (int64_t i = 0; i < Nh; ++i) t[i] = h_host[i];
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipMemcpyAsync(p->taps, t.data(), t.size() * sizeof(float),
                                  hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return FIR_OLS_ERR_HIP;
    p->has_taps = true;
    return FIR_OLS_OK;
}

int fir_pfb_execute(fir_pfb_plan_t p, const void *x_dev, void *y_dev, int64_t nsamples,
                    void *stream) {
    if (!p || nsamples < 0 || nsamples % p->D) return FIR_OLS_ERR_INVALID_ARG;
    if (!p->has_taps) return FIR_OLS_ERR_NO_FILTER;
    if (nsamples == 0) return FIR_OLS_OK;
    if (!x_dev || !y_dev || nsamples > ((int64_t)1 << 40)) return FIR_OLS_ERR_INVALID_ARG;
    if (((uintptr_t)x_dev | (uintptr_t)y_dev) & 7) return FIR_OLS_ERR_ALIGN;
    const int64_t nout = nsamples / p->D;
    const uintptr_t xa = (uintptr_t)x_dev, ya = (uintptr_t)y_dev;
    const uintptr_t xs = (uintptr_t)(nsamples * (int64_t)sizeof(float2));
    const uintptr_t ys = (uintptr_t)(nout * p->K * (int64_t)sizeof(float2));
    if (xa < ya + ys && ya < xa + xs) return FIR_OLS_ERR_ALIAS;
    if (!on_device(p)) return FIR_OLS_ERR_DEVICE;
    firpfb::PfbArgs a;
    a.x = (const float2 *)x_dev;
    a.y = (float2 *)y_dev;
    a.s_old = p->state[p->parity];
    a.s_new = p->state[p->parity ^ 1];
    a.taps = p->taps;
    a.tw = p->tw;
    a.phase = p->phase;
    a.nsamples = nsamples;
    a.nout = nout;
    a.K = p->K;
    a.D = p->D;
    a.Nh = p->Nh;
    a.TM = p->TM;
    a.t0 = (int)(p->pos % p->K);
    a.y16 = ((uintptr_t)y_dev & 15) == 0;
    if (firpfb::launch(a, p->T, p->max_groups, (hipStream_t)stream) != hipSuccess)
        return FIR_OLS_ERR_HIP;
    if (p->Nh > 1) p->parity ^= 1;
    p->pos += nsamples;
    return FIR_OLS_OK;
}

int fir_pfb_set_state(fir_pfb_plan_t p, const void *s_dev, int64_t t_next, void *stream) {
    if (!p || t_next < 0) return FIR_OLS_ERR_INVALID_ARG;
    if (s_dev && ((uintptr_t)s_dev & 7)) return FIR_OLS_ERR_ALIGN;
    if (!on_device(p)) return FIR_OLS_ERR_DEVICE;
    if (p->Nh > 1 && firols::launch_copy(p->state[p->parity], (const float2 *)s_dev, p->Nh - 1,
                                         (hipStream_t)stream) != hipSuccess)
        return FIR_OLS_ERR_HIP;
    p->pos = t_next;
    return FIR_OLS_OK;
}

int fir_pfb_get_state(fir_pfb_plan_t p, void *s_out_dev, int64_t *t_next, void *stream) {
    if (!p) return FIR_OLS_ERR_INVALID_ARG;
    if (s_out_dev && ((uintptr_t)s_out_dev & 7)) return FIR_OLS_ERR_ALIGN;
    if (!on_device(p)) return FIR_OLS_ERR_DEVICE;
    if (s_out_dev && p->Nh > 1 &&
        firols::launch_copy((float2 *)s_out_dev, p->state[p->parity], p->Nh - 1,
                            (hipStream_t)stream) != hipSuccess)
        return FIR_OLS_ERR_HIP;
    if (t_next) *t_next = p->pos;
    return FIR_OLS_OK;
}

int fir_pfb_destroy(fir_pfb_plan_t p) {
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

}  // extern "C"
