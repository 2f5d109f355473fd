// Half-resident transform of one block for any geometry of the form
// N = R0 x 1024 points, 64 points per thread (step 4 of the method page's
// claim 1): pass 0 is radix R0 (16 or 32) at stride 1024 and runs on all
// points in registers; it leaves R0 independent 1024-point sub-transforms,
// which passes 1 and 2 (radix 32 each), the product with H and inverse
// passes 2 and 1 handle in two halves of R0/2 sub-transforms, each half
// alone in LDS (N/2 points, one pad slot per 32); inverse pass 0 then runs
// on all points in registers again.
//
// With R0 = 16 (N = 16384, 256 threads) a workgroup needs about 75 KB of
// LDS and at most 256 VGPRs per thread, so two workgroups share a CU and
// one's loads and stores overlap the other's arithmetic.
//
// Layout (geometry.hpp): thread tb holds the V = 64 / R0 virtual threads
// v = tb + TB u of pass 0 (positions v + 1024 j, register R0 u + j).  In
// half h the sub-transform passes work on sub-transforms R0/2 h .. R0/2 h +
// R0/2 - 1; the LDS slot of a position p is p' + p' / 32 with
// p' = p - (N/2) h:
//   pass 0, register R0 u + j (j in [R0/2 h, R0/2 h + R0/2)):
//        v + v / 32 + 1056 (j - R0/2 h)
//   pass 1, register j:  (tb / 32) 1056 + tb % 32 + 33 j
//   pass 2, register j:  33 tb + j
// Sub-transform K of a half belongs to the 32 threads tb / 32 = K, so the
// exchanges between passes 1 and 2 stay inside half a wave.
#pragma once

#include "kernels.hpp"
#include "ols_block.hpp"

namespace firols {

template <int GID>
struct HalfRes {
    static constexpr Geo G = make_geo(GID);
    static constexpr int R0 = G.R[0];
    static constexpr int V = G.P / R0;          // virtual threads per thread in pass 0
    static constexpr int TB = G.TB;
    static constexpr int HS = R0 / 2;           // sub-transforms per half
    static constexpr int HALF = G.N / 2;
    static constexpr int HALF_SLOTS = HALF + HALF / 32;
    static constexpr int TW1 = G.S[1] * (G.R[1] - 1);   // pass-1 twiddle table in LDS
    static constexpr int NROWS = R0 == 16 ? 4 : 5;      // pass-0 twiddle rows k = 2^b
    static_assert(G.P == 64 && G.npass == 3 && (R0 == 16 || R0 == 32) && G.R[1] == 32 &&
                      G.R[2] == 32 && G.S[0] == 1024 && G.S[1] == 32 && TB % 32 == 0,
                  "half-resident layout");
};

// Twiddles: pass 0 from the plan's table (L2-resident), pass 1 from its
// copy in LDS (t = tb % 32 for every virtual thread).
template <int GID>
struct TwHalfRes {
    __amdgpu_buffer_rsrc_t tw;
    const float2 *lds_tw;
    int tb;
    template <int U, int K>
    __device__ __forceinline__ float2 operator()(ic<0>, ic<U>, ic<K>) const {
        constexpr Geo G = HalfRes<GID>::G;
        return buf_load_cached(tw, (uint32_t)tb * 8u,
                               (uint32_t)(G.twoff[0] + (K - 1) * G.S[0] + G.TB * U) * 8u);
    }
    template <int U, int K>
    __device__ __forceinline__ float2 operator()(ic<1>, ic<U>, ic<K>) const {
        return lds_tw[(K - 1) * 32 + (tb & 31)];
    }
};

template <int GID>
__device__ __forceinline__ int hr_slot0(int tb, int u) {
    return tb + (tb >> 5) + (33 * HalfRes<GID>::TB / 32) * u;
}
__device__ __forceinline__ int hr_slot1(int tb) { return (tb >> 5) * 1056 + (tb & 31); }
__device__ __forceinline__ int hr_slot2(int tb) { return 33 * tb; }

// Pass-0 registers of virtual thread U in half H to LDS and back.
template <int GID, int U, int H>
__device__ __forceinline__ void hr_put0(int tb, const float2 (&a)[64], float2 *lds) {
    using C = HalfRes<GID>;
    float2 *p = lds + hr_slot0<GID>(tb, U);
    static_for<0, C::HS>([&](auto J) {
        constexpr int j = decltype(J)::value;
        p[1056 * j] = a[C::R0 * U + C::HS * H + j];
    });
}
template <int GID, int U, int H>
__device__ __forceinline__ void hr_get0(int tb, float2 (&a)[64], const float2 *lds) {
    using C = HalfRes<GID>;
    const float2 *p = lds + hr_slot0<GID>(tb, U);
    static_for<0, C::HS>([&](auto J) {
        constexpr int j = decltype(J)::value;
        a[C::R0 * U + C::HS * H + j] = p[1056 * j];
    });
}
template <int STEP>
__device__ __forceinline__ void hr_put_run(float2 *p, const float2 (&c)[32]) {
    static_for<0, 32>([&](auto J) { p[STEP * decltype(J)::value] = c[decltype(J)::value]; });
}
template <int STEP>
__device__ __forceinline__ void hr_get_run(const float2 *p, float2 (&c)[32]) {
    static_for<0, 32>([&](auto I) {
        constexpr int j = dft_input_order<32>(decltype(I)::value);
        c[j] = p[STEP * j];
    });
}

// Radix-32 pass SI (1 or 2) of virtual thread U on 32 registers; only pass
// 1 has twiddles after it.
template <int SI, int U, class TW>
__device__ __forceinline__ void hr_fwd_vt(float2 (&c)[32], const TW &tw) {
    dft<32, -1>(c);
    if constexpr (SI == 1) {
        static_for<1, 32>([&](auto Kk) {
            c[decltype(Kk)::value] = cmul(c[decltype(Kk)::value], tw(ic<1>{}, ic<U>{}, Kk));
        });
    }
}
template <int SI, int U, class TW>
__device__ __forceinline__ void hr_inv_vt(float2 (&c)[32], const TW &tw) {
    if constexpr (SI == 1) {
        static_for<1, 32>([&](auto Kk) {
            c[decltype(Kk)::value] = cmulc(c[decltype(Kk)::value], tw(ic<1>{}, ic<U>{}, Kk));
        });
    }
    dft<32, 1>(c);
}

// Pass-0 twiddle rows W^(v 2^b), b < NROWS, of virtual thread U: a thread
// loads them once per block run and forms every other W^(v k) from them.
template <int GID, int U, class TW>
__device__ __forceinline__ void hr_load_rows(float2 (&r)[HalfRes<GID>::NROWS], const TW &tw) {
    static_for<0, HalfRes<GID>::NROWS>([&](auto Bb) {
        r[decltype(Bb)::value] = tw(ic<0>{}, ic<U>{}, ic<(1 << decltype(Bb)::value)>{});
    });
}
template <int GID, class TW>
__device__ __forceinline__ void hr_reload_rows(float2 (&r)[HalfRes<GID>::V][HalfRes<GID>::NROWS],
                                               const TW &tw) {
    TW t = tw;
    asm volatile("" : "+v"(t.tb));
    static_for<0, HalfRes<GID>::V>([&](auto Uu) {
        hr_load_rows<GID, decltype(Uu)::value>(r[decltype(Uu)::value], t);
    });
}

// Pass-0 twiddles of outputs K0 .. K1-1 of virtual thread U: with k = 4 i +
// j, W^(v k) = W^(4 v i) W^(v j), where W^(v j) (j < 4) and W^(4 v i) are
// rows or products of two or three rows.
template <int GID, int U, int K0, int K1, bool CONJ>
__device__ __forceinline__ void hr_pass0_twiddles(float2 (&a)[64],
                                                  const float2 (&r)[HalfRes<GID>::NROWS]) {
    constexpr int R0 = HalfRes<GID>::R0;
    __builtin_amdgcn_sched_barrier(0);
    const float2 l3 = cmul(r[0], r[1]);     // W^(3v)
    static_for<(K0 >> 2), ((K1 - 1) >> 2) + 1>([&](auto Ii) {
        constexpr int i = decltype(Ii)::value;
        float2 hi = r[0];                   // W^(4 v i), i > 0
        if constexpr (i == 1) hi = r[2];
        if constexpr (i == 2) hi = r[3];
        if constexpr (i == 3) hi = cmul(r[2], r[3]);
        if constexpr (R0 == 32) {
            if constexpr (i == 4) hi = r[4];
            if constexpr (i == 5) hi = cmul(r[4], r[2]);
            if constexpr (i == 6) hi = cmul(r[4], r[3]);
            if constexpr (i == 7) hi = cmul(r[4], cmul(r[2], r[3]));
        }
        static_for<0, 4>([&](auto Jj) {
            constexpr int j = decltype(Jj)::value;
            constexpr int k = 4 * i + j;
            if constexpr (k >= K0 && k < K1 && k > 0) {
                const float2 lo = j == 1 ? r[0] : j == 2 ? r[1] : l3;
                const float2 w = i == 0 ? lo : j == 0 ? hi : cmul(hi, lo);
                a[R0 * U + k] = CONJ ? cmulc(a[R0 * U + k], w) : cmul(a[R0 * U + k], w);
            }
        });
    });
    __builtin_amdgcn_sched_barrier(0);
}

// Passes 1 and 2 (forward), the product with H and inverse passes 2 and 1
// on half H.  H holds the half's factors in the pass-2 layout:
// H[(32 H + k) TB + tb].  pre() runs before the half's last barrier.
template <int GID, int H, class TW, class PRE>
__device__ __forceinline__ void hr_half(int tb, float2 *lds, const TW &tw,
                                        __amdgpu_buffer_rsrc_t Hp, const PRE &pre) {
    constexpr int TB = HalfRes<GID>::TB;
    float2 c[32];
    hr_get_run<33>(lds + hr_slot1(tb), c);
    hr_fwd_vt<1, H>(c, tw);
    hr_put_run<33>(lds + hr_slot1(tb), c);
    __builtin_amdgcn_sched_barrier(0);
    float2 hv[32];
    static_for<0, 32>([&](auto Kk) {
        constexpr int k = decltype(Kk)::value;
        hv[k] = buf_load_cached(Hp, (uint32_t)tb * 8u, (uint32_t)(32 * H + k) * TB * 8u);
    });
    __builtin_amdgcn_sched_barrier(0);
    wave_sync();
    hr_get_run<1>(lds + hr_slot2(tb), c);
    hr_fwd_vt<2, H>(c, tw);
    static_for<0, 32>([&](auto Kk) {
        constexpr int k = decltype(Kk)::value;
        c[k] = cmul(c[k], hv[k]);
    });
    hr_inv_vt<2, H>(c, tw);
    hr_put_run<1>(lds + hr_slot2(tb), c);
    wave_sync();
    hr_get_run<33>(lds + hr_slot1(tb), c);
    hr_inv_vt<1, H>(c, tw);
    hr_put_run<33>(lds + hr_slot1(tb), c);
    __builtin_amdgcn_sched_barrier(0);
    pre();
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
}

// Registers R0 .. R1-1 of block gb for real-pair channels (rows 2c and
// 2c + 1 of a float32 [2 nchan][stride] array are the real and imaginary
// parts of channel c): two range-checked 4-byte loads per point over the
// block's valid input, plus, for the blocks that reach into the state, one
// 8-byte load over the (complex) state; out-of-range loads read zero.
template <int GID, int R0, int R1>
__device__ __forceinline__ void hr_gather_real(const FusedArgs &A, int64_t gb, int tb,
                                               float2 (&v)[64]) {
    constexpr Geo G = HalfRes<GID>::G;
    const int64_t c = gb / A.nblk;
    const int64_t i = gb - c * A.nblk;
    const int Mm1 = A.M - 1;
    const int64_t g0 = i * A.L - Mm1;
    const int64_t xs = g0 > 0 ? g0 : 0;
    int64_t xn = A.nsamples - xs;
    xn = xn < 0 ? 0 : (xn > G.N ? G.N : xn);
    const float *x1 = (const float *)A.x + 2 * c * A.stride + xs;
    const __amdgpu_buffer_rsrc_t r1 = buf_rsrc(x1, (uint32_t)xn * 4u);
    const __amdgpu_buffer_rsrc_t r2 = buf_rsrc(x1 + A.stride, (uint32_t)xn * 4u);
    const int dx = (int)(g0 - xs) + tb;          // q + dx indexes the rows from xs
    auto ld = [](__amdgpu_buffer_rsrc_t r, uint32_t off) {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
    };
    if (g0 >= 0) {
        static_for<R0, R1>([&](auto Rr) {
            constexpr int r = decltype(Rr)::value;
            const uint32_t q = (uint32_t)(G.TB * pass0_m<GID>(r) + dx);
            v[r] = make_float2(ld(r1, q * 4u), ld(r2, q * 4u));
        });
    } else {
        const __amdgpu_buffer_rsrc_t rs = buf_rsrc(A.s0_old + c * Mm1, (uint32_t)Mm1 * 8u);
        const int ds = (int)(g0 + Mm1) + tb;     // q + ds indexes the state
        static_for<R0, R1>([&](auto Rr) {
            constexpr int r = decltype(Rr)::value;
            constexpr int q = G.TB * pass0_m<GID>(r);
            const uint32_t qx = buf_off<4>(q + dx);
            const float2 st = buf_load_cached(rs, (uint32_t)(q + ds) * 8u, 0);
            v[r] = make_float2(ld(r1, qx) + st.x, ld(r2, qx) + st.y);
        });
    }
}

// Step 4 of one block, ending in the store: a holds the gathered block in
// the pass-0 layout and r the pass-0 twiddle rows of every virtual thread
// (requested again at the end of each half, and left loaded for the next
// block); out(ic<U>, a) stores virtual thread U's R0 results (registers
// R0 U .. R0 U + R0 - 1, pass-0 layout) once they are final, and
// next(ic<U>, a) may then refill those registers.
template <int GID, class TW, class OUT, class NEXT>
__device__ __forceinline__ void hr_transform(int tb, float2 (&a)[64],
                                             float2 (&r)[HalfRes<GID>::V][HalfRes<GID>::NROWS],
                                             float2 *lds, const TW &tw,
                                             __amdgpu_buffer_rsrc_t Hp, const OUT &out,
                                             const NEXT &next) {
    using C = HalfRes<GID>;
    // forward pass 0; the first half's outputs go to LDS as soon as a
    // virtual thread is done
    static_for<0, C::V>([&](auto Uu) {
        constexpr int u = decltype(Uu)::value;
        __builtin_amdgcn_sched_barrier(0);
        dft_at<C::R0, -1, C::R0 * u>(a);
        hr_pass0_twiddles<GID, u, 1, C::HS, false>(a, r[u]);
        if constexpr (u == 0) __syncthreads();   // the previous block's LDS accesses are done
        hr_put0<GID, u, 0>(tb, a, lds);
    });
    __syncthreads();
    hr_half<GID, 0>(tb, lds, tw, Hp, [&] { hr_reload_rows<GID>(r, tw); });
    static_for<0, C::V>([&](auto Uu) { hr_get0<GID, decltype(Uu)::value, 0>(tb, a, lds); });
    static_for<0, C::V>([&](auto Uu) {
        constexpr int u = decltype(Uu)::value;
        hr_pass0_twiddles<GID, u, C::HS, C::R0, false>(a, r[u]);
    });
    __syncthreads();
    static_for<0, C::V>([&](auto Uu) { hr_put0<GID, decltype(Uu)::value, 1>(tb, a, lds); });
    __syncthreads();
    hr_half<GID, 1>(tb, lds, tw, Hp, [&] { hr_reload_rows<GID>(r, tw); });
    static_for<0, C::V>([&](auto Uu) {
        constexpr int u = decltype(Uu)::value;
        hr_get0<GID, u, 1>(tb, a, lds);
        hr_pass0_twiddles<GID, u, 1, C::R0, true>(a, r[u]);
        dft_at<C::R0, 1, C::R0 * u>(a);
        out(ic<u>{}, a);
        next(ic<u>{}, a);
    });
}

}  // namespace firols
