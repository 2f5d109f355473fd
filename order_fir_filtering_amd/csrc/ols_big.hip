// Overlap-save kernel for N = 32768: one block per workgroup of 512
// threads, 64 points per thread, three radix-32 passes, and no buffer
// outside the workgroup between the gather and the store.
//
// Per block E_i (method page, claim 1): gather E_i = {D_(i-1), B_i} with
// the carried state S0 in front of the first block (step 3); forward
// N-point FFT, product with H, inverse FFT (step 4); drop the first M-1
// points and store the L kept ones (step 5); the channel's last block
// writes the next state.
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
#include "kernels.hpp"
#include "ols_block.hpp"

namespace firols {

namespace {

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
    static_for<0, 32>([&](auto J) { c[decltype(J)::value] = p[STEP * decltype(J)::value]; });
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

// Pass 0 of virtual thread U is split by its output index k: the DFT and
// the twiddles of k < 16 (the first half's outputs) come first, the
// twiddles of k >= 16 only when the second half goes to LDS.  In the
// inverse the conjugate twiddles of each half are applied as it returns,
// and the DFT comes last.  This bounds the twiddles in flight at 16.
template <int U, int K0, int K1, bool CONJ, class TW>
__device__ __forceinline__ void pass0_twiddles(float2 (&a)[64], const TW &tw) {
    __builtin_amdgcn_sched_barrier(0);
    static_for<(K0 > 0 ? K0 : 1), K1>([&](auto Kk) {
        constexpr int k = decltype(Kk)::value;
        const float2 w = tw(ic<0>{}, ic<U>{}, Kk);
        a[32 * U + k] = CONJ ? cmulc(a[32 * U + k], w) : cmul(a[32 * U + k], w);
    });
    __builtin_amdgcn_sched_barrier(0);
}
// Forward pass 0 of virtual thread U with its twiddles of k < 16 already
// in registers (requested before the previous block's stores: memory
// operations complete in order, stores included, so a load issued after a
// burst of stores would wait for the burst).
template <int U>
__device__ __forceinline__ void fwd_pass0_first(float2 (&a)[64], const float2 (&w)[15]) {
    __builtin_amdgcn_sched_barrier(0);
    dft_at<32, -1, 32 * U>(a);
    static_for<1, 16>([&](auto Kk) {
        constexpr int k = decltype(Kk)::value;
        a[32 * U + k] = cmul(a[32 * U + k], w[k - 1]);
    });
    __builtin_amdgcn_sched_barrier(0);
}
template <int U, int K0, int N, class TW>
__device__ __forceinline__ void load_pass0_twiddles(float2 (&w)[N], const TW &tw) {
    static_for<0, N>([&](auto Ii) {
        w[decltype(Ii)::value] = tw(ic<0>{}, ic<U>{}, ic<K0 + decltype(Ii)::value>{});
    });
}

// Passes 1 and 2 (forward), the product with H and inverse passes 2 and 1
// of virtual thread H, on the half of the block that LDS holds.
template <int H, class TW>
__device__ __forceinline__ void big_half(int tb, float2 *lds, const TW &tw,
                                         __amdgpu_buffer_rsrc_t Hp) {
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
    __syncthreads();
    get_run<1>(lds + slot2(tb), c);
    fwd_vt<2, H>(c, tw);
    static_for<0, 32>([&](auto Kk) {
        constexpr int k = decltype(Kk)::value;
        c[k] = cmul(c[k], hv[k]);
    });
    inv_vt<2, H>(c, tw);
    put_run<1>(lds + slot2(tb), c);
    __syncthreads();
    get_run<33>(lds + slot1(tb), c);
    inv_vt<1, H>(c, tw);
    put_run<33>(lds + slot1(tb), c);
    __syncthreads();
}

// Step 4 of one block, ending in the store: a holds the gathered block in
// the pass-0 layout and w0, w1 the forward pass-0 twiddles of k < 16 of
// both virtual threads; out(ic<U>, a) stores virtual thread U's 32 results
// (registers 32 U .. 32 U + 31 of a, pass-0 layout) once they are final,
// and next(ic<U>, a) may then refill those registers (the next block's
// input, requested while this block finishes).  w0, w1 are reloaded for
// the next block before the last stores.
template <class TW, class OUT, class NEXT>
__device__ __forceinline__ void big_transform(int tb, float2 (&a)[64], float2 (&w0)[15],
                                              float2 (&w1)[15], float2 *lds, const TW &tw,
                                              __amdgpu_buffer_rsrc_t Hp, const OUT &out,
                                              const NEXT &next) {
    // forward pass 0; the first half's outputs go to LDS as soon as a
    // virtual thread is done
    fwd_pass0_first<0>(a, w0);
    __syncthreads();                 // the previous block's readers of LDS are done
    put0<0, 0>(tb, a, lds);
    fwd_pass0_first<1>(a, w1);
    put0<1, 0>(tb, a, lds);
    __syncthreads();
    big_half<0>(tb, lds, tw, Hp);
    // registers k < 16 take the first half's results back (conjugate
    // twiddles applied); the second half's forward twiddles follow
    get0<0, 0>(tb, a, lds);
    pass0_twiddles<0, 0, 16, true>(a, tw);
    get0<1, 0>(tb, a, lds);
    pass0_twiddles<1, 0, 16, true>(a, tw);
    pass0_twiddles<0, 16, 32, false>(a, tw);
    pass0_twiddles<1, 16, 32, false>(a, tw);
    __syncthreads();
    put0<0, 1>(tb, a, lds);
    put0<1, 1>(tb, a, lds);
    __syncthreads();
    big_half<1>(tb, lds, tw, Hp);
    get0<0, 1>(tb, a, lds);
    pass0_twiddles<0, 16, 32, true>(a, tw);
    dft_at<32, 1, 0>(a);
    // virtual thread 1's twiddles come before the stores and the next
    // block's input
    __builtin_amdgcn_sched_barrier(0);
    float2 wi[16];
    load_pass0_twiddles<1, 16>(wi, tw);
    __builtin_amdgcn_sched_barrier(0);
    out(ic<0>{}, a);
    next(ic<0>{}, a);
    get0<1, 1>(tb, a, lds);
    static_for<16, 32>([&](auto Kk) {
        constexpr int k = decltype(Kk)::value;
        a[32 + k] = cmulc(a[32 + k], wi[k - 16]);
    });
    dft_at<32, 1, 32>(a);
    __builtin_amdgcn_sched_barrier(0);
    load_pass0_twiddles<0, 1>(w0, tw);
    load_pass0_twiddles<1, 1>(w1, tw);
    __builtin_amdgcn_sched_barrier(0);
    out(ic<1>{}, a);
    next(ic<1>{}, a);
}

}  // namespace

__global__ __launch_bounds__(kBig.TB) void ols_big_kernel(FusedArgs A) {
    __shared__ float2 lds[kHalfSlots + kTw1];
    float2 *lds_tw = lds + kHalfSlots;
    const int tb = threadIdx.x;
    for (int e = tb; e < kTw1; e += kBig.TB) lds_tw[e] = A.tw[kBig.twoff[1] + e];
    // (the first barrier of the transform orders these writes before use)
    const int64_t units = A.nblk * A.nchan;
    // software-pipelined over blocks: the input of the next block is
    // requested as soon as the registers of a virtual thread are free
    int64_t gb = unit_of(units, blockIdx.x, gridDim.x, 0);
    float2 a[kBig.P], w0[15], w1[15];
    if (gb >= 0) {
        gather_block_wave<kBigGid, true>(A, gb, tb, a);
        const TwBig tw0{buf_rsrc(A.tw, (uint32_t)kBig.twoff[kBig.npass] * 8u), lds_tw, tb};
        load_pass0_twiddles<0, 1>(w0, tw0);
        load_pass0_twiddles<1, 1>(w1, tw0);
    }
    for (int64_t it = 1; gb >= 0; ++it) {
        const int64_t gn = unit_of(units, blockIdx.x, gridDim.x, it);
        // table pointers re-derived per block so their loads stay in the loop
        const float2 *twp = A.tw, *hp = A.H;
        asm volatile("" : "+s"(twp), "+s"(hp));
        // step 5: outputs i L .. i L + L - 1 are positions M-1 .. N-1; the
        // descriptor covers the valid outputs only, so the dropped
        // positions (negative offsets) and those past the end fall outside
        const int64_t c = gb / A.nblk;
        const int64_t i = gb - c * A.nblk;
        const int Mm1 = A.M - 1;
        int64_t yn = A.nsamples - i * A.L;
        if (yn > A.L) yn = A.L;
        const __amdgpu_buffer_rsrc_t ry =
            buf_rsrc(A.y + c * A.stride + i * A.L, (uint32_t)yn * 8u);
        const int qo = tb - Mm1;
        const __amdgpu_buffer_rsrc_t rtw = buf_rsrc(twp, (uint32_t)kBig.twoff[kBig.npass] * 8u);
        const __amdgpu_buffer_rsrc_t rh = buf_rsrc(hp, (uint32_t)kBig.N * 8u);
        big_transform(
            tb, a, w0, w1, lds, TwBig{rtw, lds_tw, tb}, rh,
            [&](auto Uu, const float2(&v)[64]) {
                constexpr int u = decltype(Uu)::value;
                static_for<0, 32>([&](auto J) {
                    constexpr int r = 32 * u + decltype(J)::value;
                    buf_store(v[r], ry, (uint32_t)(qo + kBig.TB * pass0_m<kBigGid>(r)) * 8u);
                });
            },
            [&](auto Uu, float2(&v)[64]) {
                constexpr int u = decltype(Uu)::value;
                if (gn >= 0) gather_block_wave<kBigGid, true, 32 * u, 32 * u + 32>(A, gn, tb, v);
            });
        if (i == A.nblk - 1)
            carry_state<kBigGid>(A.nsamples, Mm1, tb, A.x + c * A.stride, A.s0_old + c * Mm1,
                                 A.s0_new + c * Mm1);
        gb = gn;
    }
}

// H[r * TB + tb] = DFT_N(taps)[bin] / N in the kernel's order: the
// forward half of the transform above, one workgroup.
__global__ __launch_bounds__(kBig.TB) void ols_big_plan_taps_kernel(
    const float2 *__restrict__ taps, float2 *__restrict__ H, const float2 *__restrict__ tw) {
    __shared__ float2 lds[kHalfSlots];
    const int tb = threadIdx.x;
    const TwTable<kBigGid> twt{tw, tb};
    float2 a[kBig.P];
    static_for<0, kBig.P>([&](auto Rr) {
        constexpr int r = decltype(Rr)::value;
        a[r] = taps[tb + kBig.TB * pass0_m<kBigGid>(r)];
    });
    float2 w[15];
    load_pass0_twiddles<0, 1>(w, twt);
    fwd_pass0_first<0>(a, w);
    put0<0, 0>(tb, a, lds);
    load_pass0_twiddles<1, 1>(w, twt);
    fwd_pass0_first<1>(a, w);
    put0<1, 0>(tb, a, lds);
    constexpr float scale = 1.0f / kBig.N;
    static_for<0, 2>([&](auto Hh) {
        constexpr int h = decltype(Hh)::value;
        if constexpr (h == 1) {
            pass0_twiddles<0, 16, 32, false>(a, twt);
            pass0_twiddles<1, 16, 32, false>(a, twt);
            __syncthreads();
            put0<0, 1>(tb, a, lds);
            put0<1, 1>(tb, a, lds);
        }
        __syncthreads();
        float2 c[32];
        get_run<33>(lds + slot1(tb), c);
        fwd_vt<1, h>(c, twt);
        put_run<33>(lds + slot1(tb), c);
        __syncthreads();
        get_run<1>(lds + slot2(tb), c);
        fwd_vt<2, h>(c, twt);
        static_for<0, 32>([&](auto Kk) {
            constexpr int k = decltype(Kk)::value;
            H[(32 * h + k) * kBig.TB + tb] = make_float2(c[k].x * scale, c[k].y * scale);
        });
    });
}

int big_geometry() { return kBigGid; }

int big_max_groups(int device) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
        cus < 1)
        cus = 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, ols_big_kernel, kBig.TB, 0) !=
            hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    return cus * per_cu;
}

hipError_t launch_big(const FusedArgs &a, int max_groups, hipStream_t stream) {
    const int64_t units = a.nblk * a.nchan;
    if (units <= 0) return hipErrorInvalidConfiguration;
    int64_t grid = units;
    if (grid > max_groups) grid = max_groups & ~7;    // persistent, multiple of 8
    if (grid <= 0) grid = units < max_groups ? units : max_groups;
    hipLaunchKernelGGL(ols_big_kernel, dim3((unsigned)grid), dim3(kBig.TB), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_big_plan_taps(const float2 *taps, float2 *H, const float2 *tw,
                                hipStream_t stream) {
    hipLaunchKernelGGL(ols_big_plan_taps_kernel, dim3(1), dim3(kBig.TB), 0, stream, taps, H, tw);
    return hipGetLastError();
}

}  // namespace firols
