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
// The transform itself (ols_big.hpp) keeps half of the block in LDS at
// a time; the block never leaves the workgroup between gather and store.
#include "ols_big.hpp"

namespace firols {

// Staggered start.  Every workgroup alternates between a memory phase
// (its stores, the next block's gather) and a compute phase about twice as
// long; started together, all CUs reach their memory phase at the same
// time and share the HBM bandwidth, while a CU alone could move its data
// about twice as fast.  So when every workgroup has several blocks to do,
// the workgroups of each XCD start in three groups, 10 us apart (about a
// quarter of a block period), and the groups' memory phases interleave
// from then on (measured at M = 8193: 302 us per call without, 289 with
// two groups 16 us apart, 281 with three groups 10 us apart).
constexpr int kStaggerGroups = 3;
constexpr uint64_t kStaggerTicks = 1000;   // 10 us of the 100 MHz constant clock
constexpr int kStaggerMinBlocks = 3;       // blocks per workgroup for the stagger to pay

// REAL: the channels are pairs of real float32 rows, gathered by
// hr_gather_real and stored as two float rows.
template <bool REAL>
__global__ __launch_bounds__(kBig.TB) void ols_big_kernel(FusedArgs A) {
    __shared__ float2 lds[kHalfSlots + kTw1];
    float2 *lds_tw = lds + kHalfSlots;
    const int tb = threadIdx.x;
    for (int e = tb; e < kTw1; e += kBig.TB) lds_tw[e] = A.tw[kBig.twoff[1] + e];
    // (the first barrier of the transform orders these writes before use)
    const int64_t units = A.nblk * A.nchan;
    if ((gridDim.x & 7) == 0 && units >= (int64_t)kStaggerMinBlocks * gridDim.x) {
        // (blockIdx.x >> 3 numbers the workgroups within one XCD)
        const uint64_t wait = (uint64_t)((blockIdx.x >> 3) % kStaggerGroups) * kStaggerTicks;
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        while (__builtin_amdgcn_s_memrealtime() - t0 < wait) __builtin_amdgcn_s_sleep(8);
    }
    // software-pipelined over blocks: the input of the next block is
    // requested as soon as the registers of a virtual thread are free
    int64_t gb = unit_of(units, blockIdx.x, gridDim.x, 0);
    float2 a[kBig.P];
    BigRows r;
    if (gb >= 0) {
        if constexpr (REAL)
            hr_gather_real<kBigGid, 0, kBig.P>(A, gb, tb, a);
        else
            gather_block_wave<kBigGid, true, false>(A, gb, tb, a);
        const TwBig tw0{buf_rsrc(A.tw, (uint32_t)kBig.twoff[kBig.npass] * 8u), lds_tw, tb};
        load_big_rows(r, tw0);
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
        float *y1 = (float *)A.y + 2 * c * A.stride + i * A.L;
        const __amdgpu_buffer_rsrc_t ry1 = buf_rsrc(y1, (uint32_t)yn * 4u);
        const __amdgpu_buffer_rsrc_t ry2 = buf_rsrc(y1 + A.stride, (uint32_t)yn * 4u);
        const int qo = tb - Mm1;
        const __amdgpu_buffer_rsrc_t rtw = buf_rsrc(twp, (uint32_t)kBig.twoff[kBig.npass] * 8u);
        const __amdgpu_buffer_rsrc_t rh = buf_rsrc(hp, (uint32_t)kBig.N * 8u);
        big_transform(
            tb, a, r, lds, TwBig{rtw, lds_tw, tb}, rh,
            [&](auto Uu, const float2(&v)[64]) {
                constexpr int u = decltype(Uu)::value;
                const int qu = fresh_v(qo);
                static_for<0, 32>([&](auto J) {
                    constexpr int r = 32 * u + decltype(J)::value;
                    const int q = qu + kBig.TB * pass0_m<kBigGid>(r);
                    if constexpr (REAL) {
                        buf_store_f32(v[r].x, ry1, buf_off<4>(q));
                        buf_store_f32(v[r].y, ry2, buf_off<4>(q));
                    } else {
                        buf_store(v[r], ry, buf_off<8>(q));
                    }
                });
            },
            [&](auto Uu, float2(&v)[64]) {
                constexpr int u = decltype(Uu)::value;
                if (gn >= 0) {
                    if constexpr (REAL)
                        hr_gather_real<kBigGid, 32 * u, 32 * u + 32>(A, gn, tb, v);
                    else
                        gather_block_wave<kBigGid, true, false, 32 * u, 32 * u + 32>(A, gn, tb, v);
                }
            });
        if (i == A.nblk - 1)
            carry_state<kBigGid>(A.nsamples, Mm1, tb, ChanIn<REAL>(A, c), A.s0_old + c * Mm1,
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
    float2 r[5];
    hr_load_rows<kBigGid, 0>(r, twt);
    dft_at<32, -1, 0>(a);
    hr_pass0_twiddles<kBigGid, 0, 1, 16, false>(a, r);
    hr_put0<kBigGid, 0, 0>(tb, a, lds);
    hr_pass0_twiddles<kBigGid, 0, 16, 32, false>(a, r);
    hr_load_rows<kBigGid, 1>(r, twt);
    dft_at<32, -1, 32>(a);
    hr_pass0_twiddles<kBigGid, 1, 1, 16, false>(a, r);
    hr_put0<kBigGid, 1, 0>(tb, a, lds);
    hr_pass0_twiddles<kBigGid, 1, 16, 32, false>(a, r);
    constexpr float scale = 1.0f / kBig.N;
    static_for<0, 2>([&](auto Hh) {
        constexpr int h = decltype(Hh)::value;
        if constexpr (h == 1) {
            __syncthreads();
            hr_put0<kBigGid, 0, 1>(tb, a, lds);
            hr_put0<kBigGid, 1, 1>(tb, a, lds);
        }
        __syncthreads();
        float2 c[32];
        hr_get_run<33>(lds + hr_slot1(tb), c);
        hr_fwd_vt<1, h>(c, twt);
        hr_put_run<33>(lds + hr_slot1(tb), c);
        __syncthreads();
        hr_get_run<1>(lds + hr_slot2(tb), c);
        hr_fwd_vt<2, h>(c, twt);
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
    // the plan's workgroup count serves both variants: the smaller occupancy
    int per_cu_real = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, ols_big_kernel<false>, kBig.TB,
                                                     0) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_real, ols_big_kernel<true>, kBig.TB,
                                                     0) == hipSuccess &&
        per_cu_real >= 1 && per_cu_real < per_cu)
        per_cu = per_cu_real;
    return cus * per_cu;
}

hipError_t launch_big(const FusedArgs &a, int max_groups, hipStream_t stream, bool real) {
    const int64_t units = a.nblk * a.nchan;
    if (units <= 0) return hipErrorInvalidConfiguration;
    int64_t grid = units;
    if (grid > max_groups) grid = max_groups & ~7;    // persistent, multiple of 8
    if (grid <= 0) grid = units < max_groups ? units : max_groups;
    if (real)
        hipLaunchKernelGGL(ols_big_kernel<true>, dim3((unsigned)grid), dim3(kBig.TB), 0, stream, a);
    else
        hipLaunchKernelGGL(ols_big_kernel<false>, dim3((unsigned)grid), dim3(kBig.TB), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_big_plan_taps(const float2 *taps, float2 *H, const float2 *tw,
                                hipStream_t stream) {
    hipLaunchKernelGGL(ols_big_plan_taps_kernel, dim3(1), dim3(kBig.TB), 0, stream, taps, H, tw);
    return hipGetLastError();
}

}  // namespace firols
