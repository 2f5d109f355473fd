// Internal interface between the C ABI (plan.cpp) and the HIP kernels:
// the launch and table-building functions (host side).  The argument
// structures and size limits the kernels are compiled against are in
// kernel_args.hpp.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernel_args.hpp"

namespace firols {

// The table builders take a geometry id (geo_id(logn, logp)); a plain
// log2(N) selects the default geometry of that size.
// Twiddle table size (float2) of the transform of geometry gid.
int twiddle_count(int gid);
// Fill the twiddle table (host memory), computed in double, rounded to float.
void build_twiddles(int gid, float2 *host_out);
// perm[i]: the spectrum bin whose value the kernels expect at H[i].
void build_h_permutation(int gid, int64_t *perm);

// Geometry id of the fused kernel for a transform of 2^logn points.
int fused_geometry(int logn);
// Workgroups of the filtering kernel that fit on the device at once
// (resident workgroups per CU times CUs); the kernel is persistent and
// never launches more.
int fused_max_groups(int logn, int device);
// Filter one call (steps 3-5 of the method and the state carry).
// real: the channels are pairs of real float32 rows (a.x, a.y point to
// [2 nchan][a.stride] floats), filtered by a real response.
hipError_t launch_fused(int logn, const FusedArgs &a, int max_groups, hipStream_t stream,
                        bool real = false);
// H[i] = DFT_N(taps)[perm[i]] / N from N zero-padded complex taps.
hipError_t launch_plan_taps(int logn, const float2 *taps_padded, float2 *H,
                            const float2 *tw, hipStream_t stream);
// Half-resident kernel for N = 2^kBigLogN: its geometry id (for the
// table builders), resident workgroups, launches.
int big_geometry();
int big_max_groups(int device);
hipError_t launch_big(const FusedArgs &a, int max_groups, hipStream_t stream, bool real = false);
hipError_t launch_big_plan_taps(const float2 *taps_padded, float2 *H, const float2 *tw,
                                hipStream_t stream);
// Half-resident kernel for N = 2^kMidLogN (two workgroups per CU): its
// geometry id, resident workgroups, launches.
int mid_geometry();
int mid_max_groups(int device);
hipError_t launch_mid(const FusedArgs &a, int max_groups, hipStream_t stream, bool real = false);
hipError_t launch_mid_plan_taps(const float2 *taps_padded, float2 *H, const float2 *tw,
                                hipStream_t stream);
// Split path (N = 65536): radix of the split (N / 32768; 1 when
// N <= 2^kBigLogN), twiddle tables, H order, workgroups, launches.
int split_radix(int logn);
// H of a plan with N = 2^logn >= 65536 from N zero-padded complex taps, in
// the split / multi-pass order (scaled by 1/N).
hipError_t launch_split_plan_taps(int logn, const float2 *taps_padded, float2 *H,
                                  const float2 *tw, hipStream_t stream);
int split_sub_twiddle_count();
int64_t split_top_twiddle_count(int logn);
void build_split_twiddles(int logn, float2 *sub_tw, float2 *top_tw);
void build_split_h_permutation(int logn, int64_t *perm);
int64_t split_slot_elems(int logn);
int split_max_groups(int device);
hipError_t launch_split(int logn, const SplitArgs &a, int max_groups, hipStream_t stream,
                        bool real = false);
// Paired path (N = 65536, blocks with L valid outputs): work queues (one
// per XCD id seen on the device), resident workgroups, and the launches of
// one call (a counter reset and the kernel per batch of units).
int pair_queue_count(int device);
int pair_lead();
bool pair_hold_ready();
uint64_t pair_wait_ticks(bool hold);
int pair_max_groups(int device);
hipError_t launch_pair(const PairArgs &a, int max_groups, hipStream_t stream, bool real = false);

// Multi-pass path (N = 2^17 .. 2^20): top-pass twiddle table size and
// builder (the sub-transform shares the split path's tables and H order),
// units per batch for the plan's scratch, workgroups of the sub-transform
// kernel, and one batch's three launches.
int64_t multi_top_twiddle_count(int logn);
void build_multi_top_twiddles(int logn, float2 *top_tw);
int multi_batch_units(int logn);
int multi_max_groups(int device);
// batch_units: blocks per batch, at most what the scratch holds.
hipError_t launch_multi(int logn, const MultiArgs &a, int max_groups, int64_t batch_units,
                        hipStream_t stream, bool real = false);

// dst[i] = src ? src[i] : 0 for i < count.
hipError_t launch_copy(float2 *dst, const float2 *src, int64_t count,
                       hipStream_t stream);

}  // namespace firols
