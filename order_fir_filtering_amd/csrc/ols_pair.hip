// Overlap-save for N = 65536 with each block's two 32768-point
// sub-convolutions on two workgroups of one XCD.
//
// With Ns = N / 2, n = q + j Ns and k = k0 + 2 k' (a decimation in
// frequency by two):
//   a_k0[q] = W_N^{q k0} (E[q] + (-1)^k0 E[q + Ns]),  X[k0 + 2 k'] = DFT_Ns(a_k0)[k']
//   c_k0 = IDFT_Ns(X_k0 * H_k0),                    H_k0[k'] = H[k0 + 2 k']
//   R[q + j Ns] = c_0[q] + (-1)^j W_N^{-q} c_1[q]
// (method page, claim 1: the gathered block E_i with the carried state in
// front, step 3; FFT, product with H and inverse FFT, step 4; the first
// M-1 points of R dropped and the L others kept, step 5).
//
// Work is handed out per XCD: the blocks of a launch are split into one
// contiguous range per XCD id, and a workgroup takes items from the range
// of the XCD it runs on (hardware register XCC_ID) through an atomic
// counter, in groups: half 0 of `lead` consecutive blocks, then half 1 of
// the same blocks.  Each item
// gathers the whole block (E[q] and E[q + Ns]; the partner's second read
// of the same lines finds part of them in the shared L2 or the last-level
// cache) and runs one sub-convolution on the half-resident 32768-point
// transform (ols_big.hpp).
//  * Half 0 (the producer) parks c_0[q] in the block's own output range at
//    the position of R[q + Ns] (offset q + Ns - (M-1), always a kept point:
//    all 32768 of them lie in [Ns - (M-1), L)), waits until those stores
//    have reached L2, and raises the block's flag.
//  * Half 1 (the consumer) waits for the flag, reads c_0[q] back from L2
//    and stores R[q] (if kept) and R[q + Ns], the latter over the parked
//    value it has just read (same thread, same address).
// The producer took its item before the consumer took its own, so
// it is running, and nothing it does after that waits on another
// workgroup: the consumer's wait always ends.  It is also bounded in time;
// a wait that runs out sets the plan's error word and stores NaN instead
// of combining.  Producer and consumer run on the same XCD, so the parked
// values pass through that XCD's L2, the point of coherence between them
// (their non-temporal stores also write them back to memory, which the
// output stores then overwrite).  A queue whose XCD got no workgroup is
// run, after all other workgroups are done, by the last workgroup to
// finish, both halves of each block in turn.
//
// Only blocks whose L outputs are all valid go this way (the parked values
// need the whole output range); a call's partial last block goes through
// the one-workgroup split kernel (ols_split.hip).  Real-pair channels (two
// real rows per channel) take the same path with 4-byte row accesses.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <mutex>
#include <vector>

#include "ols_big.hpp"

namespace firols {

namespace {

constexpr int kNs = kBig.N;                      // points of a sub-transform
constexpr uint64_t kReadyWaitTicks = 50000000;   // 0.5 s of the 100 MHz constant clock
constexpr uint64_t kHeldWaitTicks = 1000;        // 10 us: the bound under FIROLS_PAIR_HOLD_READY
constexpr int kPairLead = 10;                    // default lead (measured best of 1 .. 64)

// XCD (XCC) the wave runs on: hardware register XCC_ID, bits 3:0.
__device__ __forceinline__ int xcc_id() {
    return (int)(__builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 15);
}

// Load that misses the CU's vector L1 and reads L2 (cache-policy bit sc0):
// for values another CU of the same XCD has stored.  It also carries the
// non-temporal bit: the parked values are read once (with the parking
// stores also non-temporal, the 65536-point workload ran 1.89 -> 1.86 ms
// per call against default-policy parking).
__device__ __forceinline__ float2 buf_load_l2(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
    return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 3));
}

// Wait until every vector memory access of this wave has completed (its
// stores written to L2): s_waitcnt vmcnt(0).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// The block's output range: complex channels (one descriptor over
// [nchan][stride] complex64) or real-pair channels (rows 2c and 2c + 1 of
// a float32 [2 nchan][stride] array, the real and imaginary parts).  Both
// hold L values per block, so the exchange parks c_0 in the same positions
// either way (the real-pair form splits each value over the two rows).
// Offsets outside [0, L) are dropped by the descriptors (negative ones
// through buf_off, which keeps them clear of the in-range offsets).
template <bool REAL>
struct PairOut;
template <>
struct PairOut<false> {
    __amdgpu_buffer_rsrc_t ry;
    __device__ __forceinline__ PairOut(const PairArgs &A, int64_t c, int64_t i)
        : ry(buf_rsrc(A.y + c * A.stride + i * A.L, (uint32_t)A.L * 8u)) {}
    __device__ __forceinline__ void store(float2 v, int off) const {
        buf_store(v, ry, buf_off<8>(off));
    }
    __device__ __forceinline__ float2 load_parked(int off) const {
        return buf_load_l2(ry, buf_off<8>(off));
    }
};
template <>
struct PairOut<true> {
    __amdgpu_buffer_rsrc_t r1, r2;
    __device__ __forceinline__ PairOut(const PairArgs &A, int64_t c, int64_t i) {
        float *y1 = (float *)A.y + 2 * c * A.stride + i * A.L;
        r1 = buf_rsrc(y1, (uint32_t)A.L * 4u);
        r2 = buf_rsrc(y1 + A.stride, (uint32_t)A.L * 4u);
    }
    __device__ __forceinline__ void store(float2 v, int off) const {
        buf_store_f32(v.x, r1, buf_off<4>(off));
        buf_store_f32(v.y, r2, buf_off<4>(off));
    }
    __device__ __forceinline__ float2 load_parked(int off) const {
        // sc0 + nt, as buf_load_l2
        return make_float2(
            __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r1, buf_off<4>(off), 0, 3)),
            __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r2, buf_off<4>(off), 0, 3)));
    }
};

// a_k of one block in the pass-0 layout (register r <-> q = tb + TB m):
// a_0[q] = E[q] + E[q + Ns], a_1[q] = W_N^q (E[q] - E[q + Ns]), reading
// E[q + j Ns] through load(j, q - tb); W_N^q = W_N^tb W_N^{TB m}, the
// second factor from the LDS table wm.  The loads are software-pipelined:
// kGatherAhead point pairs are in flight, and each pair consumed requests
// the next one.  A shallow pipeline is enough: the gathers of many
// workgroups at once load the memory system, not one CU's latency (on the
// 65536-point workload 28 pairs: 1.99 ms per call, 12: 1.96, 8 and 4:
// 1.956), and it leaves the compiler registers (fewer spills).
constexpr int kGatherAhead = 8;
template <bool HALF1, class LOAD>
__device__ __forceinline__ void pair_gather(float2 (&a)[64], const LOAD &load, float2 wt,
                                            const float2 *wm) {
    constexpr int D = kGatherAhead;
    float2 hi[D];
    static_for<0, D>([&](auto Rr) {
        constexpr int r = decltype(Rr)::value;
        constexpr int off = kBig.TB * pass0_m<kBigGid>(r);
        a[r] = load(0, off);
        hi[r] = load(1, off);
    });
    static_for<0, 64>([&](auto Rr) {
        constexpr int r = decltype(Rr)::value;
        __builtin_amdgcn_sched_barrier(0);
        const float2 e = hi[r % D];
        if constexpr (HALF1)
            a[r] = cmul(csub(a[r], e), cmul(wt, wm[pass0_m<kBigGid>(r)]));
        else
            a[r] = cadd(a[r], e);
        if constexpr (r + D < 64) {
            constexpr int off = kBig.TB * pass0_m<kBigGid>(r + D);
            a[r + D] = load(0, off);
            hi[(r + D) % D] = load(1, off);
        }
    });
    __builtin_amdgcn_sched_barrier(0);
}

// The consumer's combine for virtual thread U (registers 32 U .. 32 U + 31):
// c_1 in a, c_0 parked at offset off + fo of the block's output range
// (fo = tb + Ns - (M-1)); R[q] = c_0 + W_N^{-q} c_1 to offset off + qo
// (qo = tb - (M-1); dropped when negative) and R[q + Ns] =
// c_0 - W_N^{-q} c_1 over the parked value.  kCombineAhead parked values
// are in flight.
constexpr int kCombineAhead = 16;
template <int U, class OUT>
__device__ __forceinline__ void pair_combine(const float2 (&a)[64], int qo, int fo,
                                             const OUT &out, float2 wt, const float2 *wm) {
    constexpr int D = kCombineAhead;
    float2 c0[D];
    static_for<0, D>([&](auto Ii) {
        constexpr int i = decltype(Ii)::value;
        constexpr int off = kBig.TB * pass0_m<kBigGid>(32 * U + i);
        c0[i] = out.load_parked(off + fo);
    });
    static_for<0, 32>([&](auto Ii) {
        constexpr int i = decltype(Ii)::value;
        constexpr int r = 32 * U + i;
        constexpr int off = kBig.TB * pass0_m<kBigGid>(r);
        __builtin_amdgcn_sched_barrier(0);
        const float2 b1 = cmulc(a[r], cmul(wt, wm[pass0_m<kBigGid>(r)]));
        const float2 t = c0[i % D];
        out.store(cadd(t, b1), off + qo);
        out.store(csub(t, b1), off + fo);
        if constexpr (i + D < 32) {
            constexpr int off2 = kBig.TB * pass0_m<kBigGid>(r + D);
            c0[(i + D) % D] = out.load_parked(off2 + fo);
        }
    });
    __builtin_amdgcn_sched_barrier(0);
}

// What a consumer whose wait for c_0 timed out stores for virtual thread U
// instead of pair_combine's values: a quiet NaN at every kept position.
template <int U, class OUT>
__device__ __forceinline__ void pair_fill_nan(int qo, int fo, const OUT &out) {
    const float2 nan = make_float2(__builtin_nanf(""), __builtin_nanf(""));
    static_for<0, 32>([&](auto Ii) {
        constexpr int off = kBig.TB * pass0_m<kBigGid>(32 * U + decltype(Ii)::value);
        out.store(nan, off + qo);
        out.store(nan, off + fo);
    });
}

// Block (c, i) of unit u, and the offset g0 of its first point in the
// channel's input (negative: the state is in front).
struct PairBlock {
    int64_t c, i, g0;
    __device__ __forceinline__ PairBlock(const PairArgs &A, int64_t u) {
        // 32-bit division whenever the values fit (always, in practice)
        if (((uint64_t)u | (uint64_t)A.nfull) >> 32 == 0) {
            c = (uint32_t)u / (uint32_t)A.nfull;
        } else {
            c = u / A.nfull;
        }
        i = u - c * A.nfull;
        g0 = i * A.L - (A.M - 1);
    }
};

// One item: half HALF1 of unit u (block i of channel c); `ready` is the
// unit's flag; wt = W_N^tb and wm the table W_N^{TB m}.  REAL: the
// channels are real-pair rows (see PairOut), read with two 4-byte loads
// per point.
template <bool HALF1, bool REAL>
__device__ __forceinline__ void pair_item(const PairArgs &A, int64_t u, unsigned *ready, int tb,
                                          float2 *lds, const float2 *lds_tw, BigRows &r,
                                          float2 wt, const float2 *wm) {
    // (the empty asm keeps the compiler from hoisting the 64 twiddle
    // products W_N^tb W_N^{TB m}, which do not depend on the item, out of
    // the item loop into spilled registers)
    asm volatile("" : "+v"(wt.x), "+v"(wt.y));
    const PairBlock blk(A, u);
    const int64_t c = blk.c, i = blk.i, g0 = blk.g0;
    const int Mm1 = A.M - 1;
    const float2 *__restrict__ sc = A.s0_old + c * Mm1;
    // table pointers re-derived per item so their loads stay in the loop
    const float2 *twp = A.tw, *hp = A.H;
    asm volatile("" : "+s"(twp), "+s"(hp));
    const __amdgpu_buffer_rsrc_t rtw = buf_rsrc(twp, (uint32_t)kBig.twoff[kBig.npass] * 8u);
    const __amdgpu_buffer_rsrc_t rh = buf_rsrc(hp + (HALF1 ? kNs : 0), (uint32_t)kNs * 8u);

    // input sample g of the channel: complex, or the two rows' floats
    const float2 *__restrict__ xc = A.x + c * A.stride;
    const float *__restrict__ x1 = (const float *)A.x + 2 * c * A.stride;
    auto ld32 = [](__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
    };
    float2 a[64];
    if (g0 >= 0) {
        // a full block lies inside the input: g0 + N = (i + 1) L <= nsamples
        if constexpr (REAL) {
            const __amdgpu_buffer_rsrc_t r1 = buf_rsrc(x1 + g0, (uint32_t)(2 * kNs) * 4u);
            const __amdgpu_buffer_rsrc_t r2 =
                buf_rsrc(x1 + A.stride + g0, (uint32_t)(2 * kNs) * 4u);
            const uint32_t vo = (uint32_t)tb * 4u;
            pair_gather<HALF1>(a, [&](int j, int off) {
                const uint32_t so = (uint32_t)(off + j * kNs) * 4u;
                return make_float2(ld32(r1, vo, so), ld32(r2, vo, so));
            }, wt, wm);
        } else {
            const __amdgpu_buffer_rsrc_t rx = buf_rsrc(xc + g0, (uint32_t)(2 * kNs) * 8u);
            const uint32_t vo = (uint32_t)tb * 8u;
            pair_gather<HALF1>(a, [&](int j, int off) {
                return buf_load_cached(rx, vo, (uint32_t)(off + j * kNs) * 8u);
            }, wt, wm);
        }
    } else {
        // the first blocks, with the state in front: range-checked loads
        // over the input and over the (complex) state; at most one of them
        // is in range, the other reads zero
        int64_t xn = A.nsamples < 2 * kNs ? A.nsamples : 2 * kNs;
        const __amdgpu_buffer_rsrc_t rs = buf_rsrc(sc, (uint32_t)Mm1 * 8u);
        const int dx = (int)g0 + tb;           // q + dx indexes x
        const int ds = (int)(g0 + Mm1) + tb;   // q + ds indexes the state
        if constexpr (REAL) {
            const __amdgpu_buffer_rsrc_t r1 = buf_rsrc(x1, (uint32_t)xn * 4u);
            const __amdgpu_buffer_rsrc_t r2 = buf_rsrc(x1 + A.stride, (uint32_t)xn * 4u);
            pair_gather<HALF1>(a, [&](int j, int off) {
                const int q = off + j * kNs;
                const float2 st = buf_load_cached(rs, (uint32_t)(q + ds) * 8u, 0);
                return make_float2(ld32(r1, buf_off<4>(q + dx), 0) + st.x,
                                   ld32(r2, buf_off<4>(q + dx), 0) + st.y);
            }, wt, wm);
        } else {
            const __amdgpu_buffer_rsrc_t rx = buf_rsrc(xc, (uint32_t)xn * 8u);
            pair_gather<HALF1>(a, [&](int j, int off) {
                const int q = off + j * kNs;
                const float2 v = buf_load_cached(rx, buf_off<8>(q + dx), 0);
                const float2 s = buf_load_cached(rs, (uint32_t)(q + ds) * 8u, 0);
                return make_float2(v.x + s.x, v.y + s.y);
            }, wt, wm);
        }
    }

    // the block's output range.  The per-item bases go through an empty asm
    // so the 64 offsets derived from them are not hoisted out of the item
    // loop into spilled registers.
    const PairOut<REAL> out(A, c, i);
    int qo = tb - Mm1;
    int fo = tb + kNs - Mm1;
    asm volatile("" : "+v"(qo), "+v"(fo));
    if constexpr (!HALF1) {
        // producer: each virtual thread's c_0 is parked as soon as it is
        // final, with non-temporal stores (read once, by the consumer)
        big_transform(tb, a, r, lds, TwBig{rtw, lds_tw, tb}, rh,
                      [&](auto Uu, const float2(&v)[64]) {
                          constexpr int U = decltype(Uu)::value;
                          static_for<0, 32>([&](auto J) {
                              constexpr int r = 32 * U + decltype(J)::value;
                              constexpr int off = kBig.TB * pass0_m<kBigGid>(r);
                              out.store(v[r], off + fo);
                          });
                      },
                      [](auto, float2(&)[64]) {});
        wait_vmem();
        __syncthreads();
        if (tb == 0 && !A.hold_ready)
            __hip_atomic_store(ready, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        // consumer: wait for c_0 when the first virtual thread's c_1 is
        // final, combine it while the transform finishes the second one.
        // The wait is bounded; when it runs out, the plan's error word is
        // set and the block's outputs become NaN instead of a combine with
        // whatever the output range holds.
        __shared__ int sh_ok;
        int ok = 1;
        big_transform(tb, a, r, lds, TwBig{rtw, lds_tw, tb}, rh,
                      [&](auto Uu, const float2(&v)[64]) {
                          constexpr int U = decltype(Uu)::value;
                          if constexpr (U == 0) {
                              if (tb == 0) {
                                  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
                                  int got = 0;
                                  for (;;) {
                                      if (__hip_atomic_load(ready, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT) != 0u) {
                                          got = 1;
                                          break;
                                      }
                                      if (__builtin_amdgcn_s_memrealtime() - t0 >= A.wait_ticks)
                                          break;
                                      __builtin_amdgcn_s_sleep(2);
                                  }
                                  if (!got)
                                      __hip_atomic_store(A.err, 1u, __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
                                  sh_ok = got;
                              }
                              __syncthreads();
                              ok = __builtin_amdgcn_readfirstlane(sh_ok);
                          }
                          if (ok)
                              pair_combine<U>(v, qo, fo, out, wt, wm);
                          else
                              pair_fill_nan<U>(qo, fo, out);
                      },
                      [](auto, float2(&)[64]) {});
        if (i == A.nblk - 1)
            carry_state<kBigGid>(A.nsamples, Mm1, tb, ChanIn<REAL>(A, c), sc,
                                 A.s0_new + c * Mm1);
    }
}

}  // namespace

template <bool REAL>
__global__ __launch_bounds__(kBig.TB) void ols_pair_kernel(PairArgs A) {
    __shared__ float2 lds[kHalfSlots + kTw1];
    __shared__ int sh_word;
    float2 *lds_tw = lds + kHalfSlots;
    const int tb = threadIdx.x;
    __shared__ float2 wm[64];
    for (int e = tb; e < kTw1; e += kBig.TB) lds_tw[e] = A.tw[kBig.twoff[1] + e];
    // W_N^q = W_N^tb W_N^{TB m} for the points q = tb + TB m of a thread
    if (tb < 64) wm[tb] = A.tw_top[kNs + kBig.TB * tb];
    const float2 wt = A.tw_top[kNs + tb];
    // (the first barrier of the item loop orders these writes before use)
    BigRows rows;
    {
        const TwBig tw0{buf_rsrc(A.tw, (uint32_t)kBig.twoff[kBig.npass] * 8u), lds_tw, tb};
        load_big_rows(rows, tw0);
    }
    unsigned *heads = A.sync;
    unsigned *ready = A.sync + kPairSyncHeader;
    const int64_t chunk = (A.nu + A.nq - 1) / A.nq;
    // Serve the queue of this XCD until it is empty; then count this
    // workgroup out, and if it is the last one, serve every queue that is
    // not empty yet (one whose XCD had no workgroup), alone.
    int qx = xcc_id();
    bool draining = false;
    for (;;) {
        if (qx >= A.nq) {
            if (draining) break;
            __syncthreads();
            if (tb == 0)
                sh_word = __hip_atomic_fetch_add(A.sync + kPairExitWord, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1;
            __syncthreads();
            if (!__builtin_amdgcn_readfirstlane(sh_word)) break;
            draining = true;
            qx = 0;
        }
        const int64_t lo = (int64_t)qx * chunk;
        int64_t n = A.nu - lo;
        n = n < 0 ? 0 : (n > chunk ? chunk : n);
        __syncthreads();
        if (tb == 0)
            sh_word = (int)__hip_atomic_fetch_add(heads + qx, 1u, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        // the same value in every lane: make it a scalar (the block's
        // addresses and buffer descriptors derive from it)
        const int64_t j = __builtin_amdgcn_readfirstlane(sh_word);
        if (j >= 2 * n) {
            qx = draining ? qx + 1 : A.nq;
            continue;
        }
        // items come in groups of 2 lead: the producers of `lead` blocks,
        // then their consumers (fewer blocks in a queue's last group)
        const int64_t grp = j / (2 * A.lead);
        const int64_t r = j - grp * 2 * A.lead;
        const int64_t base = grp * A.lead;
        const int64_t nb = n - base < A.lead ? n - base : A.lead;
        const bool consumer = r >= nb;
        const int64_t u = lo + base + (consumer ? r - nb : r);
        if (consumer)
            pair_item<true, REAL>(A, A.u0 + u, ready + u, tb, lds, lds_tw, rows, wt, wm);
        else
            pair_item<false, REAL>(A, A.u0 + u, ready + u, tb, lds, lds_tw, rows, wt, wm);
    }
}

namespace {

__global__ __launch_bounds__(256) void zero_words_kernel(unsigned *__restrict__ p, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}

__global__ __launch_bounds__(64) void xcc_probe_kernel(int *__restrict__ out) {
    if (threadIdx.x == 0) out[blockIdx.x] = xcc_id();
}

std::mutex g_nq_mu;
int g_nq[64] = {};

}  // namespace

int pair_queue_count(int device) {
    // FIROLS_PAIR_QUEUES=n (1 .. 16) replaces the probe: with more queues
    // than XCDs, the last workgroup runs the queues no XCD serves (the
    // tests use it to exercise that path)
    if (const char *env = std::getenv("FIROLS_PAIR_QUEUES")) {
        const int n = std::atoi(env);
        if (n >= 1 && n <= kPairMaxQueues) return n;
    }
    if (device < 0 || device >= 64) return 1;
    std::lock_guard<std::mutex> lock(g_nq_mu);
    if (g_nq[device] > 0) return g_nq[device];
    // record the XCD id of many workgroups; queues cover ids 0 .. max
    constexpr int kProbe = 4096;
    int *d = nullptr;
    int nq = 0;
    if (hipMalloc(&d, kProbe * sizeof(int)) == hipSuccess) {
        hipLaunchKernelGGL(xcc_probe_kernel, dim3(kProbe), dim3(64), 0, nullptr, d);
        std::vector<int> h(kProbe, 0);
        if (hipGetLastError() == hipSuccess &&
            hipMemcpy(h.data(), d, kProbe * sizeof(int), hipMemcpyDeviceToHost) == hipSuccess)
            nq = 1 + *std::max_element(h.begin(), h.end());
        (void)hipFree(d);
    }
    (void)hipGetLastError();
    if (nq < 1 || nq > kPairMaxQueues) nq = 1;
    g_nq[device] = nq;
    return nq;
}

int pair_lead() {
    // FIROLS_PAIR_LEAD=n (1 .. 64) sets how many blocks' producers a queue
    // hands out before their consumers (a tuning knob)
    if (const char *env = std::getenv("FIROLS_PAIR_LEAD")) {
        const int n = std::atoi(env);
        if (n >= 1 && n <= 64) return n;
    }
    return kPairLead;
}

bool pair_hold_ready() {
    // FIROLS_PAIR_HOLD_READY=1 (read at plan creation) is a test switch:
    // producers raise no flag and consumers wait kHeldWaitTicks, so every
    // consumer's wait runs out and the error path can be exercised with
    // every kernel still ending normally
    const char *env = std::getenv("FIROLS_PAIR_HOLD_READY");
    return env && std::atoi(env) == 1;
}

uint64_t pair_wait_ticks(bool hold) { return hold ? kHeldWaitTicks : kReadyWaitTicks; }

int pair_max_groups(int device) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
        cus < 1)
        cus = 1;
    // the plan's workgroup count serves both variants: the smaller occupancy
    int per_cu_real = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, ols_pair_kernel<false>, kBig.TB,
                                                     0) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_real, ols_pair_kernel<true>,
                                                     kBig.TB, 0) == hipSuccess &&
        per_cu_real >= 1 && per_cu_real < per_cu)
        per_cu = per_cu_real;
    return cus * per_cu;
}

hipError_t launch_pair(const PairArgs &call, int max_groups, hipStream_t stream, bool real) {
    const int64_t units = call.nfull * call.nchan;
    if (units <= 0 || call.nq < 1 || call.nq > kPairMaxQueues || max_groups < 1)
        return hipErrorInvalidConfiguration;
    for (int64_t u0 = 0; u0 < units; u0 += kPairMaxUnits) {
        PairArgs a = call;
        a.u0 = u0;
        a.nu = (int)(units - u0 < kPairMaxUnits ? units - u0 : kPairMaxUnits);
        // every launch starts from zero counters and flags
        const int words = kPairSyncHeader + a.nu;
        hipLaunchKernelGGL(zero_words_kernel, dim3((words + 255) / 256), dim3(256), 0, stream,
                           a.sync, words);
        int64_t grid = 2 * (int64_t)a.nu;
        if (grid > max_groups) grid = max_groups;
        if (real)
            hipLaunchKernelGGL(ols_pair_kernel<true>, dim3((unsigned)grid), dim3(kBig.TB), 0,
                               stream, a);
        else
            hipLaunchKernelGGL(ols_pair_kernel<false>, dim3((unsigned)grid), dim3(kBig.TB), 0,
                               stream, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace firols
