// Per-thread phases of the LDS-resident overlap-save transform.
//
// Each function acts on the P registers of one thread (index tb within its
// block).  The kernels put a workgroup barrier between an LDS write phase
// and the read phase that follows it; see geometry.hpp for the layouts.
//
// Twiddles reach a pass through a provider `tw(ic<s>, ic<u>, ic<k>)` that
// returns W_{S R}^{t k} for pass s, virtual thread u of this thread and
// output k >= 1: either registers loaded once per kernel (loop-invariant,
// because a thread always holds the same positions of every block) or
// loads from the plan's twiddle table.
#pragma once

#include "dft.hpp"
#include "geometry.hpp"

namespace firols {

// Position held by register r in the pass-0 layout: tb + TB * m.
template <int GID>
__host__ __device__ __forceinline__ constexpr int pass0_m(int r) {
    constexpr Geo G = make_geo(GID);
    constexpr int R0 = G.R[0];
    constexpr int V0 = G.P / R0;
    return r / R0 + V0 * (r % R0);
}

// t of virtual thread u of thread tb in pass SI.
template <int GID, int SI>
__host__ __device__ __forceinline__ int pass_t(int tb, int u) {
    constexpr Geo G = make_geo(GID);
    return (tb + G.TB * u) & (G.S[SI] - 1);
}

// Number of per-thread twiddles (complex) of all passes but the last, and
// the offset of pass s among them.
template <int GID>
__host__ __device__ constexpr int thread_tw_off(int s) {
    constexpr Geo G = make_geo(GID);
    int o = 0;
    for (int i = 0; i < s && i < G.npass - 1; ++i) o += (G.P / G.R[i]) * (G.R[i] - 1);
    return o;
}
template <int GID>
__host__ __device__ constexpr int thread_tw_count() {
    return thread_tw_off<GID>(make_geo(GID).npass - 1);
}

// Twiddle provider reading the plan's table (layout: twoff[s] + (k-1)*S + t).
template <int GID>
struct TwTable {
    const float2 *__restrict__ tw;
    int tb;
    template <int SI, int U, int K>
    __host__ __device__ __forceinline__ float2 operator()(ic<SI>, ic<U>, ic<K>) const {
        constexpr Geo G = make_geo(GID);
        return tw[G.twoff[SI] + (K - 1) * G.S[SI] + pass_t<GID, SI>(tb, U)];
    }
};

// Twiddle provider holding this thread's twiddles in registers.  Only
// the rows k = 2^b of the table are read; W^(t k) for any other k is the
// product of the rows of k's set bits (k = (k & (k-1)) + lowest bit), so
// each value carries at most log2 R table roundings and log2 R - 1
// products.  A thread then reads log2 R instead of R - 1 values per pass,
// and the products run while the block's input is still in flight.
template <int GID>
struct TwRegs {
    float2 w[thread_tw_count<GID>() > 0 ? thread_tw_count<GID>() : 1];
    __host__ __device__ __forceinline__ void load(const float2 *__restrict__ tw, int tb) {
        constexpr Geo G = make_geo(GID);
        static_for<0, G.npass - 1>([&](auto Sx) {
            constexpr int s = decltype(Sx)::value;
            constexpr int R = G.R[s], V = G.P / R;
            static_for<0, V>([&](auto U) {
                constexpr int u = decltype(U)::value;
                const int t = pass_t<GID, s>(tb, u);
                static_for<1, R>([&](auto Kk) {
                    constexpr int k = decltype(Kk)::value;
                    if constexpr ((k & (k - 1)) == 0)
                        w[thread_tw_off<GID>(s) + u * (R - 1) + k - 1] =
                            tw[G.twoff[s] + (k - 1) * G.S[s] + t];
                });
            });
        });
        static_for<0, G.npass - 1>([&](auto Sx) {
            constexpr int s = decltype(Sx)::value;
            constexpr int R = G.R[s], V = G.P / R;
            static_for<0, V>([&](auto U) {
                constexpr int o = thread_tw_off<GID>(s) + decltype(U)::value * (R - 1) - 1;
                static_for<1, R>([&](auto Kk) {
                    constexpr int k = decltype(Kk)::value;
                    if constexpr ((k & (k - 1)) != 0)
                        w[o + k] = cmul(w[o + (k & (k - 1))], w[o + (k & -k)]);
                });
            });
        });
    }
    template <int SI, int U, int K>
    __host__ __device__ __forceinline__ float2 operator()(ic<SI>, ic<U>, ic<K>) const {
        constexpr int R = make_geo(GID).R[SI];
        return w[thread_tw_off<GID>(SI) + U * (R - 1) + K - 1];
    }
};

// H provider reading the plan's H (kernel order: H[r * TB + tb]).
template <int GID>
struct HTable {
    const float2 *__restrict__ H;
    int tb;
    template <int R>
    __host__ __device__ __forceinline__ float2 operator()(ic<R>) const {
        return H[R * make_geo(GID).TB + tb];
    }
};

// H provider holding this thread's P values in registers.
template <int GID>
struct HRegs {
    float2 h[make_geo(GID).P];
    __host__ __device__ __forceinline__ void load(const float2 *__restrict__ H, int tb) {
        constexpr Geo G = make_geo(GID);
        static_for<0, G.P>([&](auto Rr) {
            h[decltype(Rr)::value] = H[decltype(Rr)::value * G.TB + tb];
        });
    }
    template <int R>
    __host__ __device__ __forceinline__ float2 operator()(ic<R>) const { return h[R]; }
};

// Forward pass SI: R-point DFTs, then the inter-pass twiddles W_{S R}^{t k}.
template <int GID, int SI, class TW>
__host__ __device__ __forceinline__ void fwd_pass(float2 (&a)[make_geo(GID).P], const TW &tw) {
    constexpr Geo G = make_geo(GID);
    constexpr int R = G.R[SI], V = G.P / R;
    static_for<0, V>([&](auto U) {
        constexpr int u = decltype(U)::value;
        dft_at<R, -1, u * R>(a);
        if constexpr (SI < G.npass - 1) {
            static_for<1, R>([&](auto Kk) {
                constexpr int k = decltype(Kk)::value;
                a[u * R + k] = cmul(a[u * R + k], tw(ic<SI>{}, U, Kk));
            });
        }
    });
}

// Inverse pass SI: conjugate twiddles, then R-point inverse DFTs.
template <int GID, int SI, class TW>
__host__ __device__ __forceinline__ void inv_pass(float2 (&a)[make_geo(GID).P], const TW &tw) {
    constexpr Geo G = make_geo(GID);
    constexpr int R = G.R[SI], V = G.P / R;
    static_for<0, V>([&](auto U) {
        constexpr int u = decltype(U)::value;
        if constexpr (SI < G.npass - 1) {
            static_for<1, R>([&](auto Kk) {
                constexpr int k = decltype(Kk)::value;
                a[u * R + k] = cmulc(a[u * R + k], tw(ic<SI>{}, U, Kk));
            });
        }
        dft_at<R, 1, u * R>(a);
    });
}

// LDS slot of register j of virtual thread v in pass SI is
// lds_base(v) + j * lds_step: with one pad slot per P positions the slot
// stays linear in j because S is 1 or a multiple of P (and S*R <= P when
// S == 1).
template <int GID, int SI>
__host__ __device__ __forceinline__ int lds_base(int v) {
    constexpr Geo G = make_geo(GID);
    constexpr int R = G.R[SI], S = G.S[SI];
    static_assert(S % G.P == 0 || S * R <= G.P, "LDS slot not linear in j");
    const int base = (v / S) * (S * R) + (v & (S - 1));
    return lds_pad(G, base);
}
template <int GID, int SI>
__host__ __device__ constexpr int lds_step() {
    constexpr Geo G = make_geo(GID);
    return G.S[SI] % G.P == 0 ? G.S[SI] + G.S[SI] / G.P : G.S[SI];
}

// Store the registers of pass SI's layout into the block's LDS slots.
template <int GID, int SI>
__host__ __device__ __forceinline__ void lds_put(int tb, const float2 (&a)[make_geo(GID).P],
                                                 float2 *lds) {
    constexpr Geo G = make_geo(GID);
    constexpr int R = G.R[SI], V = G.P / R, st = lds_step<GID, SI>();
    static_for<0, V>([&](auto U) {
        constexpr int u = decltype(U)::value;
        float2 *p = lds + lds_base<GID, SI>(tb + G.TB * u);
        static_for<0, R>([&](auto J) { p[decltype(J)::value * st] = a[u * R + decltype(J)::value]; });
    });
}

// Load the registers of pass SI's layout from the block's LDS slots.
template <int GID, int SI>
__host__ __device__ __forceinline__ void lds_get(int tb, float2 (&a)[make_geo(GID).P],
                                                 const float2 *lds) {
    constexpr Geo G = make_geo(GID);
    constexpr int R = G.R[SI], V = G.P / R, st = lds_step<GID, SI>();
    static_for<0, V>([&](auto U) {
        constexpr int u = decltype(U)::value;
        const float2 *p = lds + lds_base<GID, SI>(tb + G.TB * u);
        static_for<0, R>([&](auto I) {
            constexpr int j = dft_input_order<R>(decltype(I)::value);
            a[u * R + j] = p[j * st];
        });
    });
}

// Pointwise product with H.
template <int GID, class HP>
__host__ __device__ __forceinline__ void mul_h(float2 (&a)[make_geo(GID).P], const HP &h) {
    constexpr Geo G = make_geo(GID);
    static_for<0, G.P>([&](auto Rr) {
        constexpr int r = decltype(Rr)::value;
        a[r] = cmul(a[r], h(Rr));
    });
}

}  // namespace firols
