// Device building blocks shared by the overlap-save kernels: the forward
// and inverse pass sequences with their LDS exchanges, the XCD-aware work
// order, raw buffer access and the state carry.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"
#include "ols_phases.hpp"

namespace firols {

// Barrier of an LDS exchange.  A block of at most 64 threads lies inside
// one wave, and a wave's LDS operations execute in order, so its exchange
// needs only a wave-level barrier (which keeps the compiler from moving
// LDS accesses across it); larger blocks need the workgroup barrier.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
template <int GID>
__device__ __forceinline__ void block_sync() {
    if constexpr (make_geo(GID).TB <= 64)
        wave_sync();
    else
        __syncthreads();
}

// Barrier of the exchange between passes s-1 and s.  When both passes
// have one virtual thread per thread and the same radix, the positions
// pass s reads of one sub-block of S[s-1] points were all written by the
// S[s-1] consecutive threads that own that sub-block, so with S[s-1] <= 64
// the exchange stays inside a wave.
template <int GID, int SI>
__device__ __forceinline__ void exchange_sync() {
    constexpr Geo G = make_geo(GID);
    constexpr bool local = G.TB <= 64 ||
                           (G.R[SI - 1] == G.P && G.R[SI] == G.P && G.S[SI - 1] <= 64);
    if constexpr (local)
        wave_sync();
    else
        __syncthreads();
}

// Swap one float between two registers across lane bit LB (4: the odd
// 16-lane rows of `lo` with the even rows of `hi`; 5: the upper 32 lanes of
// `lo` with the lower 32 lanes of `hi`).  Afterwards `lo` holds, at a lane
// with bit LB clear, its own old value and at a lane with bit LB set the
// old `hi` of the lane with that bit clear; `hi` the converse.
template <int LB>
__device__ __forceinline__ void row_swap(float &lo, float &hi) {
    const unsigned x = __builtin_bit_cast(unsigned, lo), y = __builtin_bit_cast(unsigned, hi);
    if constexpr (LB == 4) {
        const auto v = __builtin_amdgcn_permlane16_swap(x, y, false, false);
        lo = __builtin_bit_cast(float, (unsigned)v[0]);
        hi = __builtin_bit_cast(float, (unsigned)v[1]);
    } else {
        static_assert(LB == 5, "row swaps exist for lane bits 4 and 5");
        const auto v = __builtin_amdgcn_permlane32_swap(x, y, false, false);
        lo = __builtin_bit_cast(float, (unsigned)v[0]);
        hi = __builtin_bit_cast(float, (unsigned)v[1]);
    }
}

// Exchange from the layout of pass FROM to that of pass TO inside the
// wave's registers, when lane_swap_plan accepts it: for N = 1024 (radices
// 4, 16, 16, one wave per block) the exchange between the first two passes
// moves position bits 8, 9 from registers to lanes 4, 5 and bits 4, 5 the
// other way, i.e. two row swaps per pair of registers and no LDS round
// trip or barrier; N = 512 needs one.
template <int GID, int FROM, int TO>
__device__ __forceinline__ void lane_exchange(float2 (&a)[make_geo(GID).P]) {
    constexpr Geo G = make_geo(GID);
    constexpr LaneSwap ls = lane_swap_plan(G, FROM, TO);
    static_assert(ls.ok, "exchange is not a set of lane-row swaps");
    static_for<0, 2>([&](auto I) {
        constexpr int i = decltype(I)::value;
        constexpr int rb = ls.rb[i];
        if constexpr (rb >= 0) {
            static_for<0, G.P>([&](auto Rr) {
                constexpr int r = decltype(Rr)::value;
                if constexpr ((r & (1 << rb)) == 0) {
                    row_swap<4 + i>(a[r].x, a[r | (1 << rb)].x);
                    row_swap<4 + i>(a[r].y, a[r | (1 << rb)].y);
                }
            });
        }
    });
}

// Forward passes with exchanges between them: inside the wave's registers
// where the layouts allow it (lane_exchange), else through LDS.
template <int GID, class TW>
__device__ __forceinline__ void forward_all(int tb, float2 (&a)[make_geo(GID).P],
                                            float2 *lds, const TW &tw) {
    constexpr Geo G = make_geo(GID);
    static_for<0, G.npass>([&](auto Sx) {
        constexpr int s = decltype(Sx)::value;
        if constexpr (s > 0) {
            if constexpr (lane_swap_plan(G, s - 1, s).ok) {
                lane_exchange<GID, s - 1, s>(a);
            } else {
                block_sync<GID>();
                lds_put<GID, s - 1>(tb, a, lds);
                exchange_sync<GID, s>();
                lds_get<GID, s>(tb, a, lds);
            }
        }
        fwd_pass<GID, s>(a, tw);
    });
}

// Inverse passes in reverse order, exchanged as in forward_all.
template <int GID, class TW>
__device__ __forceinline__ void inverse_all(int tb, float2 (&a)[make_geo(GID).P],
                                            float2 *lds, const TW &tw) {
    constexpr Geo G = make_geo(GID);
    static_for<0, G.npass>([&](auto Ix) {
        constexpr int s = G.npass - 1 - decltype(Ix)::value;
        if constexpr (s < G.npass - 1) {
            if constexpr (lane_swap_plan(G, s + 1, s).ok) {
                lane_exchange<GID, s + 1, s>(a);
            } else {
                block_sync<GID>();
                lds_put<GID, s + 1>(tb, a, lds);
                exchange_sync<GID, s + 1>();
                lds_get<GID, s>(tb, a, lds);
            }
        }
        inv_pass<GID, s>(a, tw);
    });
}

// Work unit (BPW consecutive blocks) of the it-th iteration of workgroup w,
// or -1 when the workgroup is done.  Workgroups are dispatched round-robin
// over the 8 XCDs (w % 8); each XCD takes one contiguous eighth of the
// units, so neighbouring blocks, whose gathers overlap by M-1 samples, run
// on the same XCD and share its L2.
__device__ __forceinline__ int64_t unit_of(int64_t units, int w, int G, int64_t it) {
    if ((G & 7) == 0) {
        const int per = G >> 3;
        const int64_t chunk = (units + 7) >> 3;
        const int64_t lo = (int64_t)(w & 7) * chunk;
        const int64_t u = lo + (w >> 3) + it * per;
        const int64_t hi = lo + chunk < units ? lo + chunk : units;
        return u < hi ? u : -1;
    }
    const int64_t u = w + it * G;
    return u < units ? u : -1;
}

// Raw buffer access (gfx9 family): a 128-bit descriptor holds a base
// address and a byte size; a load whose 32-bit offset is at or past the
// size returns zero and such a store is dropped.  The kernels use this to
// zero-fill positions outside the input and to drop the M-1 discarded and
// the past-the-end outputs without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}
// Byte offset of element e (SIZE bytes per element) for a range-checked
// buffer access where e may be negative: a position before the buffer,
// to read as zero or to drop.  A negative e wraps to 2^32 - SIZE |e|,
// which is at least 2^31 here (|e| stays below 2^21); every byte offset at
// or above 2^30 becomes 2^30, past every buffer these accesses use (at
// most 2^20 elements of 8 bytes).  The plain wrap is not safe: a 4-byte
// access whose lanes held wrapped offsets just below 2^32 next to in-range
// lanes at 0, 4, ... read zero for those in-range lanes too (and such
// stores were dropped), when M - 1 was not a multiple of 4.  With e a
// per-thread base plus a constant this is one v_add and one v_min.
template <int SIZE>
__device__ __forceinline__ uint32_t buf_off(int e) {
    const uint32_t b = (uint32_t)e * (uint32_t)SIZE;
    return b < 0x40000000u ? b : 0x40000000u;
}

// v through an empty asm: the offsets derived from it are formed where
// they are used instead of being hoisted out of the block loop and kept
// live (64 clamped offsets per thread would spill)
__device__ __forceinline__ int fresh_v(int v) {
    asm volatile("" : "+v"(v));
    return v;
}

// Non-temporal load (cache-policy bit 1): for input that the small-block
// kernel streams through once when every workgroup has a single block
// (several blocks per workgroup measured faster with the default policy,
// which keeps the M-1 samples two neighbouring blocks share in L2 longer).
__device__ __forceinline__ float2 buf_load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 2));
}
// Default-policy load: the plan's tables (twiddles, H), which every block
// reads again, and the input of the large-block kernels, where the overlap
// with the next block is read by the same workgroup one block later (the
// non-temporal policy measured slower there).
__device__ __forceinline__ float2 buf_load_cached(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                  uint32_t soff) {
    return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
template <bool NT>
__device__ __forceinline__ float2 buf_load_policy(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                  uint32_t soff) {
    if constexpr (NT)
        return buf_load(r, voff, soff);
    else
        return buf_load_cached(r, voff, soff);
}
// Output stores carry the non-temporal policy (cache-policy bit 1, NT on
// gfx950): the outputs are not read again, and streaming them out during
// the kernel leaves fewer dirty L2 lines to write back when it ends.
constexpr int kStoreNT = 2;
__device__ __forceinline__ void buf_store(float2 v, __amdgpu_buffer_rsrc_t r, uint32_t voff) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(decltype(
        __builtin_amdgcn_raw_buffer_load_b64(r, 0, 0, 0)), v), r, voff, 0, kStoreNT);
}
// Default-policy store with a scalar offset, for scratch data that is read
// back soon (all in range).
__device__ __forceinline__ void buf_store_cached(float2 v, __amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                 uint32_t soff) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(decltype(
        __builtin_amdgcn_raw_buffer_load_b64(r, 0, 0, 0)), v), r, voff, soff, 0);
}
// Input of channel c as complex samples.  With REAL the channel is a pair
// of real rows, 2c and 2c + 1 of a float32 [2 nchan][stride] array, whose
// samples are the real and imaginary parts (two real streams filtered by a
// real filter at once: the real and imaginary parts of the output are the
// two filtered streams).
template <bool REAL>
struct ChanIn {
    const float2 *__restrict__ xc;
    const float *__restrict__ x1;
    const float *__restrict__ x2;
    template <class ARGS>   // any call's arguments with x and stride
    __device__ __forceinline__ ChanIn(const ARGS &A, int64_t c)
        : xc(A.x + c * A.stride),
          x1((const float *)A.x + 2 * c * A.stride),
          x2((const float *)A.x + (2 * c + 1) * A.stride) {}
    __device__ __forceinline__ float2 operator[](int64_t g) const {
        if constexpr (REAL)
            return make_float2(x1[g], x2[g]);
        else
            return xc[g];
    }
};

__device__ __forceinline__ float buf_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                              uint32_t soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 2));
}
__device__ __forceinline__ void buf_store_f32(float v, __amdgpu_buffer_rsrc_t r, uint32_t voff) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, voff, 0, kStoreNT);
}

// State carry: the last M-1 samples of {S0, x} of channel c go to the new
// state buffer (TB threads of the block that ends the channel); xc[g] is
// the channel's sample g (a pointer or a ChanIn).
template <int GID, class XC>
__device__ __forceinline__ void carry_state(int64_t nsamples, int Mm1, int tb, const XC &xc,
                                            const float2 *__restrict__ sc,
                                            float2 *__restrict__ sn) {
    constexpr Geo G = make_geo(GID);
    for (int r = tb; r < Mm1; r += G.TB) {
        const int64_t g = nsamples - Mm1 + r;
        sn[r] = g >= 0 ? xc[g] : sc[Mm1 + g];
    }
}

// The same block for TB >= 64: every wave belongs to one block, so the
// block's channel, index and buffer descriptors are wave-uniform (SGPRs)
// and all gathers and stores are buffer accesses with 32-bit offsets.
// Split in two so a kernel can issue a block's input loads before other
// loads it does not need yet.  With BUF_EDGE the first and last blocks
// also gather through buffer descriptors (two range-checked loads per
// point: one over the valid input, one over the state), which keeps the
// per-point address registers of large P out of the kernel.
// NT selects the input loads' cache policy; R0 .. R1 selects the
// registers to fill (default: all); REAL reads a pair of real rows per
// channel (see ChanIn).
template <int GID, bool BUF_EDGE = false, bool NT = true, int R0 = 0, int R1 = make_geo(GID).P,
          bool REAL = false>
__device__ __forceinline__ void gather_block_wave(const FusedArgs &A, int64_t gb, int tb,
                                                  float2 (&a)[make_geo(GID).P]) {
    constexpr Geo G = make_geo(GID);
    static_assert(G.TB % 64 == 0, "one block per wave or more");
    static_assert(!(REAL && BUF_EDGE), "real pairs take the pointer edge path");
    const int64_t total = A.nblk * A.nchan;
    const bool active = gb < total;
    const int64_t c = active ? gb / A.nblk : 0;
    const int64_t i = active ? gb - c * A.nblk : 0;
    const int Mm1 = A.M - 1;
    const float2 *__restrict__ xc = A.x + c * A.stride;
    const float2 *__restrict__ sc = A.s0_old + c * Mm1;
    const int64_t g0 = i * A.L - Mm1;
    if constexpr (REAL) {
        const ChanIn<true> xr(A, c);
        if (active && g0 >= 0 && g0 + G.N <= A.nsamples) {
            // interior block: two 4-byte loads per point, one per row
            const __amdgpu_buffer_rsrc_t r1 = buf_rsrc(xr.x1 + g0, G.N * 4u);
            const __amdgpu_buffer_rsrc_t r2 = buf_rsrc(xr.x2 + g0, G.N * 4u);
            const uint32_t vo = (uint32_t)tb * 4u;
            static_for<R0, R1>([&](auto Rr) {
                constexpr int r = decltype(Rr)::value;
                constexpr uint32_t so = (uint32_t)(G.TB * pass0_m<GID>(r) * 4);
                a[r] = make_float2(buf_load_f32(r1, vo, so), buf_load_f32(r2, vo, so));
            });
        } else {
            static_for<R0, R1>([&](auto Rr) {
                constexpr int r = decltype(Rr)::value;
                const int64_t g = g0 + tb + G.TB * pass0_m<GID>(r);
                float2 v = make_float2(0.f, 0.f);
                if (active) {
                    if (g < 0)
                        v = sc[Mm1 + g];
                    else if (g < A.nsamples)
                        v = xr[g];
                }
                a[r] = v;
            });
        }
        return;
    }
    if (active && g0 >= 0 && g0 + G.N <= A.nsamples) {
        // interior block: one load per point, constant offsets in SGPRs
        const __amdgpu_buffer_rsrc_t rx = buf_rsrc(xc + g0, G.N * 8u);
        const uint32_t vo = (uint32_t)tb * 8u;
        static_for<R0, R1>([&](auto Rr) {
            constexpr int r = decltype(Rr)::value;
            a[r] = buf_load_policy<NT>(rx, vo, (uint32_t)(G.TB * pass0_m<GID>(r) * 8));
        });
    } else if constexpr (BUF_EDGE) {
        // first blocks (state in front) and the partial last block: the
        // whole offset sits in the range-checked VGPR operand; at most one
        // of the two loads is in range, the other reads zero
        const int64_t xs = active && g0 > 0 ? g0 : 0;
        int64_t xn = active ? A.nsamples - xs : 0;
        xn = xn < 0 ? 0 : (xn > G.N ? G.N : xn);
        const __amdgpu_buffer_rsrc_t rx = buf_rsrc(xc + xs, (uint32_t)xn * 8u);
        const __amdgpu_buffer_rsrc_t rs =
            buf_rsrc(sc, active && g0 < 0 ? (uint32_t)Mm1 * 8u : 0u);
        const int dx = (int)(g0 - xs) + tb;     // q + dx indexes x from xs
        // q + ds indexes the state (formed in 64 bits and kept unsigned:
        // past the state, where g0 + M - 1 may not fit 32 bits, it wraps,
        // and the state descriptor is empty there)
        const uint32_t ds = (uint32_t)(g0 + Mm1 + tb);
        static_for<R0, R1>([&](auto Rr) {
            constexpr int off = G.TB * pass0_m<GID>(decltype(Rr)::value);
            const float2 u = buf_load_policy<NT>(rx, buf_off<8>(off + dx), 0);
            const float2 v = buf_load_policy<NT>(rs, ((uint32_t)off + ds) * 8u, 0);
            a[decltype(Rr)::value] = make_float2(u.x + v.x, u.y + v.y);
        });
    } else {
        // first blocks (state in front) and the partial last block
        static_for<R0, R1>([&](auto Rr) {
            constexpr int r = decltype(Rr)::value;
            const int64_t g = g0 + tb + G.TB * pass0_m<GID>(r);
            float2 v = make_float2(0.f, 0.f);
            if (active) {
                if (g < 0)
                    v = sc[Mm1 + g];
                else if (g < A.nsamples)
                    v = xc[g];
            }
            a[r] = v;
        });
    }
}

// Store of a block's kept points (step 5) from the pass-0 layout, and the
// state carry of the channel's last block.  Outputs i L .. i L + L - 1
// come from positions q = M-1 .. N-1; the descriptor covers the valid
// outputs only, so the dropped positions (negative offset) and those past
// the end fall outside it.
template <int GID, bool REAL = false>
__device__ __forceinline__ void store_block_wave(const FusedArgs &A, int64_t gb, int tb,
                                                 const float2 (&a)[make_geo(GID).P]) {
    constexpr Geo G = make_geo(GID);
    const int64_t total = A.nblk * A.nchan;
    const bool active = gb < total;
    const int64_t c = active ? gb / A.nblk : 0;
    const int64_t i = active ? gb - c * A.nblk : 0;
    const int Mm1 = A.M - 1;
    int64_t yn = active ? A.nsamples - i * A.L : 0;
    if (yn > A.L) yn = A.L;
    if (yn < 0) yn = 0;
    if constexpr (REAL) {
        // the real part to row 2c, the imaginary part to row 2c + 1
        float *y1 = (float *)A.y + 2 * c * A.stride + i * A.L;
        const __amdgpu_buffer_rsrc_t r1 = buf_rsrc(y1, (uint32_t)yn * 4u);
        const __amdgpu_buffer_rsrc_t r2 = buf_rsrc(y1 + A.stride, (uint32_t)yn * 4u);
        static_for<0, G.P>([&](auto Rr) {
            constexpr int r = decltype(Rr)::value;
            const int q = tb + G.TB * pass0_m<GID>(r);
            buf_store_f32(a[r].x, r1, buf_off<4>(q - Mm1));
            buf_store_f32(a[r].y, r2, buf_off<4>(q - Mm1));
        });
    } else {
        const __amdgpu_buffer_rsrc_t ry =
            buf_rsrc(A.y + c * A.stride + i * A.L, (uint32_t)yn * 8u);
        static_for<0, G.P>([&](auto Rr) {
            constexpr int r = decltype(Rr)::value;
            const int q = tb + G.TB * pass0_m<GID>(r);
            buf_store(a[r], ry, buf_off<8>(q - Mm1));
        });
    }

    if (active && i == A.nblk - 1)
        carry_state<GID>(A.nsamples, Mm1, tb, ChanIn<REAL>(A, c), A.s0_old + c * Mm1,
                         A.s0_new + c * Mm1);
}

}  // namespace firols
