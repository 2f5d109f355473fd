// Internal interface between the channelizer's C ABI (pfb_plan.cpp) and
// its HIP kernels (pfb.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace firpfb {

// Arguments of one channelizer call.
struct PfbArgs {
    const float2 *x;        // nsamples input samples
    float2 *y;              // [nout][K] outputs, nout = nsamples / D
    const float2 *s_old;    // Nh - 1 samples before the call (null when Nh == 1)
    float2 *s_new;          // the last Nh - 1 samples of {s_old, x}
    const float *taps;      // T * K prototype taps, zero past Nh
    const float2 *tw;       // twiddle table of the K-point transform
    const float2 *phase;    // K values exp(-2 pi j e / K)
    int64_t nsamples;
    int64_t nout;
    int K, D, Nh;
    int TM;                 // outputs per workgroup tile
    int t0;                 // stream time of x[0], mod K
    int y16;                // y is 16-byte aligned: two channels per store
};

constexpr int kMinLogK = 6;
constexpr int kMaxLogK = 10;
constexpr int kMaxTapsPerBranch = 8;

// Taps per branch the kernels take for Nh taps at K channels (2, 4 or 8),
// or 0 when Nh needs more.
int taps_per_branch(int K, int Nh);
// Outputs per tile (a multiple of the transforms a workgroup runs at once),
// or 0 when the tile's input does not fit the workgroup's LDS.
int tile_outputs(int K, int D, int T);
int twiddle_count(int K);
void build_twiddles(int K, float2 *host_out);
// Workgroups of the channelizer kernel resident on the device at once.
int max_groups(int K, int T, int device);
// One call: the channelizer kernel, then the state carry.
hipError_t launch(const PfbArgs &a, int T, int max_groups, hipStream_t stream);

}  // namespace firpfb
