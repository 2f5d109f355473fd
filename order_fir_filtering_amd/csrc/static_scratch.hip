// fir_ols_execute_static: the filtering call with the kernels' scratch
// taken from a fixed array in device memory instead of the plan's own
// allocation, for callers that cannot allocate (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array below is a device-side symbol: on the host, its name is only a
// stand-in for the symbol and is never passed to a kernel or a copy.  The
// device address of each GPU's copy is looked up once per device with
// hipGetSymbolAddress (on the first call made with that device current)
// and kept in g_ptr; the kernels receive that address.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "firols.h"
#include "kernels.hpp"
#include "plan.hpp"

namespace {

// 64 MiB: at N = 65536 the two-workgroup kernel's flags (512 KB) and 127
// slots for the one-workgroup kernel of partial last blocks; above 65536
// the blocks of one multi-pass batch (8 blocks at N = 2^20, 64 at 2^17).
constexpr int64_t kStaticScratchBytes = (int64_t)64 << 20;
constexpr int64_t kStaticScratchElems = kStaticScratchBytes / (int64_t)sizeof(float2);
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) float2 scratch[kStaticScratchElems];

namespace {

std::mutex g_mu;
float2 *g_ptr[kMaxDevices] = {};

// Device address of this device's copy of the scratch array (looked up
// once per device), or null when the lookup fails.
float2 *scratch_ptr(int device) {
    if (device < 0 || device >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[device]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_ptr[device] = static_cast<float2 *>(ptr);
    }
    return g_ptr[device];
}

}  // namespace

extern "C" int64_t fir_ols_static_scratch_bytes(void) { return kStaticScratchBytes; }

extern "C" int fir_ols_execute_static(fir_ols_plan_t p, const void *x_dev, void *y_dev,
                                      int64_t nsamples, int64_t chan_stride, void *stream) {
    if (!p) return FIR_OLS_ERR_INVALID_ARG;
    if (p->scratch_elems == 0)   // N <= 32768: these kernels use no scratch
        return firols::execute_with_scratch(p, x_dev, y_dev, nsamples, chan_stride, stream,
                                            false, nullptr, 0);
    // a block of the plan must fit the array (every N the library takes
    // does: at most 8 MiB per block)
    if (p->N > kStaticScratchElems) return FIR_OLS_ERR_UNSUPPORTED;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return FIR_OLS_ERR_HIP;
    if (dev != p->device) return FIR_OLS_ERR_DEVICE;
    float2 *s = scratch_ptr(dev);
    if (!s) return FIR_OLS_ERR_HIP;
    return firols::execute_with_scratch(p, x_dev, y_dev, nsamples, chan_stride, stream, false, s,
                                        kStaticScratchElems);
}
