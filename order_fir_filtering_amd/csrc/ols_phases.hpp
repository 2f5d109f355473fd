// Per-thread phases of the LDS-resident overlap-save transform.
//
// Each function acts on the P registers of one thread (index tb within its
// block).  The kernels put a workgroup barrier between an LDS write phase
// and the read phase that follows it; see geometry.hpp for the layouts.
#pragma once

#include "dft.hpp"
#include "geometry.hpp"

namespace firols {

// Position held by register r in the pass-0 layout: tb + TB * m.
template <int LOGN>
__host__ __device__ __forceinline__ constexpr int pass0_m(int r) {
    constexpr Geo G = make_geo(LOGN);
    constexpr int R0 = G.R[0];
    constexpr int V0 = G.P / R0;
    return r / R0 + V0 * (r % R0);
}

// Forward pass SI: R-point DFTs, then the inter-pass twiddles W_{S R}^{t k}.
template <int LOGN, int SI>
__host__ __device__ __forceinline__ void fwd_pass(int tb, float2 (&a)[make_geo(LOGN).P],
                                                  const float2 *__restrict__ tw) {
    constexpr Geo G = make_geo(LOGN);
    constexpr int R = G.R[SI], S = G.S[SI], V = G.P / R;
    static_for<0, V>([&](auto U) {
        constexpr int u = decltype(U)::value;
        dft_at<R, -1, u * R>(a);
        if constexpr (SI < G.npass - 1) {
            const int t = (tb + G.TB * u) & (S - 1);
            const float2 *w = tw + G.twoff[SI] + t;
            static_for<1, R>([&](auto Kk) {
                constexpr int k = decltype(Kk)::value;
                a[u * R + k] = cmul(a[u * R + k], w[(k - 1) * S]);
            });
        }
    });
}

// Inverse pass SI: conjugate twiddles, then R-point inverse DFTs.
template <int LOGN, int SI>
__host__ __device__ __forceinline__ void inv_pass(int tb, float2 (&a)[make_geo(LOGN).P],
                                                  const float2 *__restrict__ tw) {
    constexpr Geo G = make_geo(LOGN);
    constexpr int R = G.R[SI], S = G.S[SI], V = G.P / R;
    static_for<0, V>([&](auto U) {
        constexpr int u = decltype(U)::value;
        if constexpr (SI < G.npass - 1) {
            const int t = (tb + G.TB * u) & (S - 1);
            const float2 *w = tw + G.twoff[SI] + t;
            static_for<1, R>([&](auto Kk) {
                constexpr int k = decltype(Kk)::value;
                a[u * R + k] = cmulc(a[u * R + k], w[(k - 1) * S]);
            });
        }
        dft_at<R, 1, u * R>(a);
    });
}

// Base position of virtual thread v in pass SI.
template <int LOGN, int SI>
__host__ __device__ __forceinline__ int pass_base(int v) {
    constexpr Geo G = make_geo(LOGN);
    constexpr int R = G.R[SI], S = G.S[SI];
    return (v / S) * (S * R) + (v & (S - 1));
}

// Store the registers of pass SI's layout into the block's LDS slots.
template <int LOGN, int SI>
__host__ __device__ __forceinline__ void lds_put(int tb, const float2 (&a)[make_geo(LOGN).P],
                                                 float2 *lds) {
    constexpr Geo G = make_geo(LOGN);
    constexpr int R = G.R[SI], S = G.S[SI], V = G.P / R;
    static_for<0, V>([&](auto U) {
        constexpr int u = decltype(U)::value;
        const int base = pass_base<LOGN, SI>(tb + G.TB * u);
        static_for<0, R>([&](auto J) {
            constexpr int j = decltype(J)::value;
            lds[lds_pad(base + S * j)] = a[u * R + j];
        });
    });
}

// Load the registers of pass SI's layout from the block's LDS slots.
template <int LOGN, int SI>
__host__ __device__ __forceinline__ void lds_get(int tb, float2 (&a)[make_geo(LOGN).P],
                                                 const float2 *lds) {
    constexpr Geo G = make_geo(LOGN);
    constexpr int R = G.R[SI], S = G.S[SI], V = G.P / R;
    static_for<0, V>([&](auto U) {
        constexpr int u = decltype(U)::value;
        const int base = pass_base<LOGN, SI>(tb + G.TB * u);
        static_for<0, R>([&](auto J) {
            constexpr int j = decltype(J)::value;
            a[u * R + j] = lds[lds_pad(base + S * j)];
        });
    });
}

// Pointwise product with H (kernel order: H[r * TB + tb]).
template <int LOGN>
__host__ __device__ __forceinline__ void mul_h(int tb, float2 (&a)[make_geo(LOGN).P],
                                               const float2 *__restrict__ H) {
    constexpr Geo G = make_geo(LOGN);
    static_for<0, G.P>([&](auto Rr) {
        constexpr int r = decltype(Rr)::value;
        a[r] = cmul(a[r], H[r * G.TB + tb]);
    });
}

}  // namespace firols
