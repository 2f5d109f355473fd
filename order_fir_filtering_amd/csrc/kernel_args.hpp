// Argument structures and size limits shared by the overlap-save kernels
// and the host code that launches them.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace firols {

// Arguments of one overlap-save call over nchan channels.
struct FusedArgs {
    const float2 *x;        // [nchan][stride] input
    float2 *y;              // [nchan][stride] output
    const float2 *s0_old;   // [nchan][M-1] state read by this call (may be null if M == 1)
    float2 *s0_new;         // [nchan][M-1] state written by this call
    const float2 *H;        // N values, kernel order, scaled by 1/N
    const float2 *tw;       // twiddle table of the transform
    int64_t nsamples;       // samples per channel in this call (> 0)
    int64_t stride;         // elements between channel starts
    int64_t nblk;           // blocks per channel = ceil(nsamples / L)
    int M;                  // taps
    int L;                  // kept outputs per block
    int nchan;
};

// Arguments of one call of the split (N = 65536) path.
struct SplitArgs {
    const float2 *x;        // [nchan][stride] input
    float2 *y;              // [nchan][stride] output
    const float2 *s0_old;   // [nchan][M-1] state read by this call
    float2 *s0_new;         // [nchan][M-1] state written by this call
    const float2 *H;        // RT * Ns values: bins k0 + RT k' in sub-kernel order, / N
    const float2 *tw;       // twiddle table of the Ns-point sub-transform
    const float2 *tw_top;   // RT * Ns values W_N^{q k0}, k0 = 0 .. RT-1 (row 0 all ones)
    float2 *scratch;        // one slot of RT * Ns values per resident workgroup
    int64_t nsamples;       // samples per channel in this call (> 0)
    int64_t stride;         // elements between channel starts
    int64_t nblk;           // blocks per channel
    int64_t blk0;           // first block of every channel this launch runs (blocks blk0 .. nblk-1)
    int M;
    int L;
    int nchan;
};

// Arguments of one launch of the paired N = 65536 kernel over the units
// u0 .. u0 + nu - 1 (unit = c * nfull + i) of a call's full blocks.
struct PairArgs {
    const float2 *x;        // [nchan][stride] input
    float2 *y;              // [nchan][stride] output
    const float2 *s0_old;   // [nchan][M-1] state read by this call
    float2 *s0_new;         // [nchan][M-1] state written by this call
    const float2 *H;        // 2 * Ns values: bins k0 + 2 k' in sub-kernel order, / N
    const float2 *tw;       // twiddle table of the Ns-point sub-transform
    const float2 *tw_top;   // 2 * Ns values W_N^{q k0} (row 0 all ones)
    unsigned *sync;         // kPairSyncHeader words (queue heads, exit count), then nu flags
    unsigned *err;          // the plan's error word: set to 1 when a consumer's wait times out
    uint64_t wait_ticks;    // bound of a consumer's wait, 100 MHz constant-clock ticks
    int64_t nsamples;       // samples per channel in this call (> 0)
    int64_t stride;         // elements between channel starts
    int64_t nblk;           // blocks per channel
    int64_t nfull;          // leading blocks per channel with L valid outputs
    int64_t u0;             // first unit of the launch
    int nu;                 // units in the launch
    int nq;                 // work queues: one per XCD id 0 .. nq-1
    int lead;               // blocks whose producers a queue hands out before their consumers
    int hold_ready;         // test switch: producers park c_0 but raise no flag
    int M;
    int L;
    int nchan;
};

// Words of the paired kernel's synchronization area before the per-unit
// flags: one queue head per XCD id (at most 16), the exit count, padding.
constexpr int kPairSyncHeader = 32;
constexpr int kPairMaxQueues = 16;
constexpr int kPairExitWord = 16;
// Units per launch of the paired kernel (its flags fill 256 KB, within
// the 512 KB the split path's scratch reserves for them).
constexpr int kPairMaxUnits = 65536;
static_assert((kPairSyncHeader + kPairMaxUnits) * 4 <= 65536 * 8, "flags fit one slot");

// Arguments of one batch of the multi-pass path (N = 2^17 .. 2^20): the
// units (channel, block) u0 .. u0 + nu - 1 of a call, unit = c * nblk + i.
struct MultiArgs {
    const float2 *x;        // [nchan][stride] input
    float2 *y;              // [nchan][stride] output
    const float2 *s0_old;   // [nchan][M-1] state read by this call
    float2 *s0_new;         // [nchan][M-1] state written by this call
    const float2 *H;        // RT * Ns values: bins k0 + RT k' in sub-kernel order, / N
    const float2 *tw;       // twiddle table of the Ns-point sub-transform
    const float2 *tw_top;   // W_N^{q k0} factors: [RT][256] (q mod 256), then [RT][Ns/256]
    float2 *scratch;        // [nu][RT][Ns]: the sub-sequences, then their convolutions
    int64_t nsamples;       // samples per channel in this call (> 0)
    int64_t stride;         // elements between channel starts
    int64_t nblk;           // blocks per channel
    int64_t u0;             // first unit of the batch
    int nu;                 // units in the batch
    int M;
    int L;
    int nchan;
};

// Largest log2(N) the LDS-resident kernel covers; N = 2^kBigLogN takes the
// half-resident kernel, N = 2^kSplitLogN the split path, larger N (up to
// kMaxLogN) the multi-pass path.
constexpr int kFusedMaxLogN = 14;
constexpr int kMidLogN = 14;
constexpr int kBigLogN = 15;
constexpr int kSplitLogN = 16;
constexpr int kMaxLogN = 20;
constexpr int kMinLogN = 3;

}  // namespace firols
