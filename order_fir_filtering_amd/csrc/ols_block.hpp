// Device building blocks shared by the overlap-save kernels: the forward
// and inverse pass sequences with their LDS exchanges, the XCD-aware work
// order, raw buffer access and the state carry.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "ols_phases.hpp"

namespace firols {

// Forward passes with LDS exchanges between them.
template <int GID, class TW>
__device__ __forceinline__ void forward_all(int tb, float2 (&a)[make_geo(GID).P],
                                            float2 *lds, const TW &tw) {
    constexpr Geo G = make_geo(GID);
    static_for<0, G.npass>([&](auto Sx) {
        constexpr int s = decltype(Sx)::value;
        if constexpr (s > 0) {
            __syncthreads();
            lds_put<GID, s - 1>(tb, a, lds);
            __syncthreads();
            lds_get<GID, s>(tb, a, lds);
        }
        fwd_pass<GID, s>(a, tw);
    });
}

// Inverse passes in reverse order with LDS exchanges between them.
template <int GID, class TW>
__device__ __forceinline__ void inverse_all(int tb, float2 (&a)[make_geo(GID).P],
                                            float2 *lds, const TW &tw) {
    constexpr Geo G = make_geo(GID);
    static_for<0, G.npass>([&](auto Ix) {
        constexpr int s = G.npass - 1 - decltype(Ix)::value;
        if constexpr (s < G.npass - 1) {
            __syncthreads();
            lds_put<GID, s + 1>(tb, a, lds);
            __syncthreads();
            lds_get<GID, s>(tb, a, lds);
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
// Input loads also carry the non-temporal policy: each sample is read by
// at most two neighbouring blocks close together in time.
__device__ __forceinline__ float2 buf_load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 2));
}
// Output stores carry the non-temporal policy (cache-policy bit 1, NT on
// gfx950): the outputs are not read again, and streaming them out during
// the kernel leaves fewer dirty L2 lines to write back when it ends.
constexpr int kStoreNT = 2;
typedef float nt_float2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void nt_store(float2 *p, float2 v) {
    __builtin_nontemporal_store(nt_float2{v.x, v.y}, reinterpret_cast<nt_float2 *>(p));
}
__device__ __forceinline__ void buf_store(float2 v, __amdgpu_buffer_rsrc_t r, uint32_t voff) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(decltype(
        __builtin_amdgcn_raw_buffer_load_b64(r, 0, 0, 0)), v), r, voff, 0, kStoreNT);
}

// State carry: the last M-1 samples of {S0, x} of channel c go to the new
// state buffer (TB threads of the block that ends the channel).
template <int GID>
__device__ __forceinline__ void carry_state(int64_t nsamples, int Mm1, int tb,
                                            const float2 *__restrict__ xc,
                                            const float2 *__restrict__ sc,
                                            float2 *__restrict__ sn) {
    constexpr Geo G = make_geo(GID);
    for (int r = tb; r < Mm1; r += G.TB) {
        const int64_t g = nsamples - Mm1 + r;
        sn[r] = g >= 0 ? xc[g] : sc[Mm1 + g];
    }
}

}  // namespace firols
