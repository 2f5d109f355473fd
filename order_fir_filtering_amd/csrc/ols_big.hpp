// The 32768-point half-resident transform of one block (step 4 of the
// method page's claim 1), shared by the N = 32768 kernel and the
// sub-transforms of the N = 65536 split and of the N = 2^17 .. 2^20
// multi-pass path.
//
// The block (256 KB) does not fit the 160 KB LDS, so the transform is
// ordered around that: pass 0 (stride 1024) runs on all 32768 points in
// registers; it leaves 32 independent 1024-point sub-transforms, which
// passes 1 and 2, the product with H and inverse passes 2 and 1 handle in
// two halves of 16 sub-transforms, each half alone in LDS (16384 points
// with one pad slot per 32); inverse pass 0 then runs on all points in
// registers again.  A thread keeps at most 64 points live: the pass-0
// outputs of the half still waiting plus the 32 points it works on.
//
// Layout (see geometry.hpp): thread tb holds virtual threads v = tb and
// tb + 512 in every pass.  In half h the sub-transform passes work on
// virtual thread u = h only, and the LDS slot of a position p is
// p' + p' / 32 with p' = p - 16384 h:
//   pass 0, register 32 u + j (j in [16h, 16h+16)):  (tb + tb/32 + 528 u) + 1056 (j - 16h)
//   pass 1, register j:                               (tb/32) 1056 + tb%32 + 33 j
//   pass 2, register j:                               33 tb + j
// Passes 1 and 2 read and write back the same slots (in place), so a
// barrier is needed only where data moves between threads.
#pragma once

#include "kernels.hpp"
#include "ols_block.hpp"

namespace firols {

constexpr int kBigGid = geo_id(15, 6, 5);
constexpr Geo kBig = make_geo(kBigGid);
static_assert(kBig.P == 64 && kBig.TB == 512 && kBig.npass == 3 && kBig.R[0] == 32 &&
                  kBig.R[1] == 32 && kBig.R[2] == 32 && kBig.S[1] == 32,
              "layout of the half-resident transform");
constexpr int kHalf = kBig.N / 2;
constexpr int kHalfSlots = kHalf + kHalf / 32;
constexpr int kTw1 = kBig.S[1] * (kBig.R[1] - 1);   // pass-1 twiddle table in LDS

// Twiddles: pass 0 from the plan's table (L2-resident), pass 1 from its
// copy in LDS (t = tb % 32 for both virtual threads).
// The table loads are buffer loads with the thread's offset in the VGPR
// operand and the constant part in the scalar one (all in range).
struct TwBig {
    __amdgpu_buffer_rsrc_t tw;
    const float2 *lds_tw;
    int tb;
    template <int U, int K>
    __device__ __forceinline__ float2 operator()(ic<0>, ic<U>, ic<K>) const {
        return buf_load_cached(tw, (uint32_t)tb * 8u,
                               (uint32_t)(kBig.twoff[0] + (K - 1) * kBig.S[0] + kBig.TB * U) * 8u);
    }
    template <int U, int K>
    __device__ __forceinline__ float2 operator()(ic<1>, ic<U>, ic<K>) const {
        return lds_tw[(K - 1) * kBig.S[1] + (tb & (kBig.S[1] - 1))];
    }
};

__device__ __forceinline__ int slot0(int tb, int u) { return tb + (tb >> 5) + 528 * u; }
__device__ __forceinline__ int slot1(int tb) { return (tb >> 5) * 1056 + (tb & 31); }
__device__ __forceinline__ int slot2(int tb) { return 33 * tb; }

// Pass-0 registers of virtual thread U in half H (j in [16H, 16H+16)) to
// LDS and back.
template <int U, int H>
__device__ __forceinline__ void put0(int tb, const float2 (&a)[64], float2 *lds) {
    float2 *p = lds + slot0(tb, U);
    static_for<0, 16>([&](auto J) {
        constexpr int j = decltype(J)::value;
        p[1056 * j] = a[32 * U + 16 * H + j];
    });
}
template <int U, int H>
__device__ __forceinline__ void get0(int tb, float2 (&a)[64], const float2 *lds) {
    const float2 *p = lds + slot0(tb, U);
    static_for<0, 16>([&](auto J) {
        constexpr int j = decltype(J)::value;
        a[32 * U + 16 * H + j] = p[1056 * j];
    });
}
template <int STEP>
__device__ __forceinline__ void put_run(float2 *p, const float2 (&c)[32]) {
    static_for<0, 32>([&](auto J) { p[STEP * decltype(J)::value] = c[decltype(J)::value]; });
}
template <int STEP>
__device__ __forceinline__ void get_run(const float2 *p, float2 (&c)[32]) {
    static_for<0, 32>([&](auto I) {
        constexpr int j = dft_input_order<32>(decltype(I)::value);
        c[j] = p[STEP * j];
    });
}

// Forward / inverse radix-32 pass SI of virtual thread U on 32 registers.
template <int SI, int U, class TW>
__device__ __forceinline__ void fwd_vt(float2 (&c)[32], const TW &tw) {
    dft<32, -1>(c);
    if constexpr (SI < kBig.npass - 1) {
        static_for<1, 32>([&](auto Kk) {
            c[decltype(Kk)::value] = cmul(c[decltype(Kk)::value], tw(ic<SI>{}, ic<U>{}, Kk));
        });
    }
}
template <int SI, int U, class TW>
__device__ __forceinline__ void inv_vt(float2 (&c)[32], const TW &tw) {
    if constexpr (SI < kBig.npass - 1) {
        static_for<1, 32>([&](auto Kk) {
            c[decltype(Kk)::value] = cmulc(c[decltype(Kk)::value], tw(ic<SI>{}, ic<U>{}, Kk));
        });
    }
    dft<32, 1>(c);
}

// Pass-0 twiddles W^(t k) (t = tb + 512 U, k in [1, 32)) of virtual
// thread U are formed in registers from the five table rows k = 1, 2, 4,
// 8, 16, which a thread loads once and keeps for all its blocks (they do
// not depend on the block): with k = 4 i + j, W^(t k) = W^(4 t i) W^(t j),
// where W^(t j) (j < 4) and W^(4 t i) (i < 8) are rows or products of
// two or three rows.  Each value carries at most five table roundings and
// four products.
template <int U, class TW>
__device__ __forceinline__ void load_pass0_rows(float2 (&r)[5], const TW &tw) {
    static_for<0, 5>([&](auto Bb) {
        r[decltype(Bb)::value] = tw(ic<0>{}, ic<U>{}, ic<(1 << decltype(Bb)::value)>{});
    });
}
// The rows are requested again where they are needed after a phase that
// holds many registers (the empty asm makes the request a new one, so the
// compiler does not keep the earlier values live across that phase).
template <class TW>
__device__ __forceinline__ void reload_pass0_rows(float2 (&r0)[5], float2 (&r1)[5], const TW &tw) {
    TW t = tw;
    asm volatile("" : "+v"(t.tb));
    load_pass0_rows<0>(r0, t);
    load_pass0_rows<1>(r1, t);
}
// Pass 0 of virtual thread U is split by its output index k: the DFT and
// the twiddles of k < 16 (the first half's outputs) come first, the
// twiddles of k >= 16 only when the second half goes to LDS.  In the
// inverse all conjugate twiddles are applied just before the last DFT.
// pass0_twiddles applies the twiddles of outputs K0 .. K1-1.
template <int U, int K0, int K1, bool CONJ>
__device__ __forceinline__ void pass0_twiddles(float2 (&a)[64], const float2 (&r)[5]) {
    __builtin_amdgcn_sched_barrier(0);
    const float2 l3 = cmul(r[0], r[1]);     // W^(3t)
    static_for<(K0 >> 2), ((K1 - 1) >> 2) + 1>([&](auto Ii) {
        constexpr int i = decltype(Ii)::value;
        float2 hi = r[0];                   // W^(4 t i), i > 0
        if constexpr (i == 1) hi = r[2];
        if constexpr (i == 2) hi = r[3];
        if constexpr (i == 3) hi = cmul(r[2], r[3]);
        if constexpr (i == 4) hi = r[4];
        if constexpr (i == 5) hi = cmul(r[4], r[2]);
        if constexpr (i == 6) hi = cmul(r[4], r[3]);
        if constexpr (i == 7) hi = cmul(r[4], cmul(r[2], r[3]));
        static_for<0, 4>([&](auto Jj) {
            constexpr int j = decltype(Jj)::value;
            constexpr int k = 4 * i + j;
            if constexpr (k >= K0 && k < K1 && k > 0) {
                const float2 lo = j == 1 ? r[0] : j == 2 ? r[1] : l3;
                const float2 w = i == 0 ? lo : j == 0 ? hi : cmul(hi, lo);
                a[32 * U + k] = CONJ ? cmulc(a[32 * U + k], w) : cmul(a[32 * U + k], w);
            }
        });
    });
    __builtin_amdgcn_sched_barrier(0);
}
// Forward pass 0 of virtual thread U with the twiddles of k < 16.
template <int U>
__device__ __forceinline__ void fwd_pass0_first(float2 (&a)[64], const float2 (&r)[5]) {
    __builtin_amdgcn_sched_barrier(0);
    dft_at<32, -1, 32 * U>(a);
    pass0_twiddles<U, 1, 16, false>(a, r);
}

// Passes 1 and 2 (forward), the product with H and inverse passes 2 and 1
// of virtual thread H, on the half of the block that LDS holds.
// pre() runs before the half's last barrier, when its working registers
// are free (the caller requests loads it needs right after the half).
template <int H, class TW, class PRE>
__device__ __forceinline__ void big_half(int tb, float2 *lds, const TW &tw,
                                         __amdgpu_buffer_rsrc_t Hp, const PRE &pre) {
    // Sub-transform K of the half belongs to the 32 threads tb / 32 = K, and
    // its pass-1 and pass-2 slots both lie in [1056 K, 1056 K + 1056): the
    // exchanges between passes 1 and 2 stay inside half a wave, so a wave
    // barrier orders them and the waves run this part independently.
    float2 c[32];
    get_run<33>(lds + slot1(tb), c);
    fwd_vt<1, H>(c, tw);
    put_run<33>(lds + slot1(tb), c);
    // this half's H is requested before the barrier, so its latency
    // overlaps the wait and the pass-2 DFT
    __builtin_amdgcn_sched_barrier(0);
    float2 hv[32];
    static_for<0, 32>([&](auto Kk) {
        constexpr int k = decltype(Kk)::value;
        hv[k] = buf_load_cached(Hp, (uint32_t)tb * 8u, (uint32_t)(32 * H + k) * kBig.TB * 8u);
    });
    __builtin_amdgcn_sched_barrier(0);
    wave_sync();
    get_run<1>(lds + slot2(tb), c);
    fwd_vt<2, H>(c, tw);
    static_for<0, 32>([&](auto Kk) {
        constexpr int k = decltype(Kk)::value;
        c[k] = cmul(c[k], hv[k]);
    });
    inv_vt<2, H>(c, tw);
    put_run<1>(lds + slot2(tb), c);
    wave_sync();
    get_run<33>(lds + slot1(tb), c);
    inv_vt<1, H>(c, tw);
    put_run<33>(lds + slot1(tb), c);
    __builtin_amdgcn_sched_barrier(0);
    pre();
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
}

// Step 4 of one block, ending in the store: a holds the gathered block in
// the pass-0 layout and r0, r1 the pass-0 twiddle rows of both virtual
// threads (requested again at the end of each half, and left loaded for
// the next block); out(ic<U>, a) stores virtual thread U's 32 results
// (registers 32 U .. 32 U + 31 of a, pass-0 layout) once they are final,
// and next(ic<U>, a) may then refill those registers (the next block's
// input, requested while this block finishes).
template <class TW, class OUT, class NEXT>
__device__ __forceinline__ void big_transform(int tb, float2 (&a)[64], float2 (&r0)[5],
                                              float2 (&r1)[5], float2 *lds, const TW &tw,
                                              __amdgpu_buffer_rsrc_t Hp, const OUT &out,
                                              const NEXT &next) {
    // forward pass 0; the first half's outputs go to LDS as soon as a
    // virtual thread is done
    fwd_pass0_first<0>(a, r0);
    __syncthreads();                 // the previous block's LDS accesses are done
    put0<0, 0>(tb, a, lds);
    fwd_pass0_first<1>(a, r1);
    put0<1, 0>(tb, a, lds);
    __syncthreads();
    // the first half's results wait untwiddled in registers k < 16 until
    // the last DFT
    big_half<0>(tb, lds, tw, Hp, [&] { reload_pass0_rows(r0, r1, tw); });
    get0<0, 0>(tb, a, lds);
    get0<1, 0>(tb, a, lds);
    pass0_twiddles<0, 16, 32, false>(a, r0);
    pass0_twiddles<1, 16, 32, false>(a, r1);
    __syncthreads();
    put0<0, 1>(tb, a, lds);
    put0<1, 1>(tb, a, lds);
    __syncthreads();
    big_half<1>(tb, lds, tw, Hp, [&] { reload_pass0_rows(r0, r1, tw); });
    get0<0, 1>(tb, a, lds);
    pass0_twiddles<0, 1, 32, true>(a, r0);
    dft_at<32, 1, 0>(a);
    out(ic<0>{}, a);
    next(ic<0>{}, a);
    get0<1, 1>(tb, a, lds);
    pass0_twiddles<1, 1, 32, true>(a, r1);
    dft_at<32, 1, 32>(a);
    out(ic<1>{}, a);
    next(ic<1>{}, a);
}

}  // namespace firols
