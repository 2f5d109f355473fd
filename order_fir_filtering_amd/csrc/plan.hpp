// The plan object behind the C ABI's opaque handle (shared by the
// library's host sources; not part of the public interface).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

struct fir_ols_plan_s {
    int device = 0;
    int logn = 0;
    int64_t M = 0, N = 0, L = 0, nchan = 0;
    float2 *H = nullptr;          // N values, kernel order, scaled by 1/N
    float2 *tw = nullptr;         // twiddle table
    float2 *taps = nullptr;       // N zero-padded taps, staging for set_taps
    float2 *state[2] = {nullptr, nullptr};   // [nchan][M-1] each
    int parity = 0;               // state[parity] is the current state
    int max_groups = 0;           // resident workgroups of the filtering kernel
    bool has_filter = false;
    bool real_filter = false;     // the filter came from real taps (set_taps, is_complex == 0)
    // split path (N = 65536) and multi-pass path (N = 2^17 .. 2^20)
    float2 *tw_top = nullptr;     // W_N^{q k0} (split: full rows; multi-pass: two factors)
    float2 *scratch = nullptr;    // split: max_groups slots of N values; multi-pass: a batch of blocks
    int64_t scratch_elems = 0;    // float2 values at scratch
    int pair_nq = 0;              // split path: work queues of the paired kernel (XCD ids)
    int pair_groups = 0;          // split path: resident workgroups of the paired kernel
    int pair_lead = 10;           // split path: producers handed out ahead of their consumers
    bool pair_hold = false;       // split path: test switch FIROLS_PAIR_HOLD_READY (no flags raised)
    unsigned *err = nullptr;      // device word: 1 after a kernel wait ran out (fir_ols_check)
    // host-resident streaming (fir_ols_execute_host), created on first use
    int64_t hs_chunk = 0;                      // samples per channel of a staging slot
    float2 *hs_x[2] = {nullptr, nullptr};      // device input slots [nchan][hs_chunk]
    float2 *hs_y[2] = {nullptr, nullptr};      // device output slots [nchan][hs_chunk]
    hipStream_t hs_in = nullptr, hs_out = nullptr;   // copy streams (default priority)
    hipEvent_t hs_ev[8] = {};                  // in[2], comp[2], out[2], start, end
};

// Frees the host-streaming resources of a plan (no-op when never used).
void release_host_stream(fir_ols_plan_s *p);

namespace firols {
// The filtering call behind fir_ols_execute (real == false) and
// fir_ols_execute_real (real == true), with the kernels' scratch area given
// explicitly (scratch_elems float2 values; only the N >= 65536 paths use
// it).  Argument checks and status codes as fir_ols_execute;
// FIR_OLS_ERR_UNSUPPORTED when the scratch cannot hold one N-sample slot.
int execute_with_scratch(fir_ols_plan_s *p, const void *x_dev, void *y_dev, int64_t nsamples,
                         int64_t stride, void *stream, bool real, float2 *scratch,
                         int64_t scratch_elems);
}  // namespace firols
