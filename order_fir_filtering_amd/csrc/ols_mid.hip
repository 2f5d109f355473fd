// Overlap-save kernel for N = 16384: one block per workgroup of 256
// threads, 64 points per thread (a radix-16 pass, then two radix-32 passes
// on 1024-point sub-transforms, half of the block in LDS at a time), two
// workgroups per CU.
//
// Per block E_i (method page, claim 1): gather E_i = {D_(i-1), B_i} with
// the carried state S0 in front of the first block (step 3); forward
// N-point FFT, product with H, inverse FFT (step 4); drop the first M-1
// points and store the L kept ones (step 5); the channel's last block
// writes the next state.
//
// A workgroup needs 75 KB of LDS and at most 256 VGPRs per thread, so a CU
// holds two: while one gathers or stores, the other computes, which one
// workgroup per CU (the 32768-point kernel) cannot do.
#include "ols_halfres.hpp"

namespace firols {

namespace {

constexpr int kMidGid = geo_id(14, 6, 5);
using Mid = HalfRes<kMidGid>;
static_assert(Mid::TB == 256 && Mid::R0 == 16 && Mid::V == 4, "N = 16384 layout");

}  // namespace

// REAL: the channels are pairs of real float32 rows (gathered by
// hr_gather_real, stored as two float rows).
template <bool REAL>
__global__ __launch_bounds__(Mid::TB, 2) void ols_mid_kernel(FusedArgs A) {
    constexpr Geo G = Mid::G;
    __shared__ float2 lds[Mid::HALF_SLOTS + Mid::TW1];
    float2 *lds_tw = lds + Mid::HALF_SLOTS;
    const int tb = threadIdx.x;
    for (int e = tb; e < Mid::TW1; e += Mid::TB) lds_tw[e] = A.tw[G.twoff[1] + e];
    // (the first barrier of the transform orders these writes before use)
    const int64_t units = A.nblk * A.nchan;
    // software-pipelined over blocks: the input of the next block is
    // requested as soon as the registers of a virtual thread are free
    int64_t gb = unit_of(units, blockIdx.x, gridDim.x, 0);
    float2 a[G.P], r[Mid::V][Mid::NROWS];
    if (gb >= 0) {
        if constexpr (REAL)
            hr_gather_real<kMidGid, 0, G.P>(A, gb, tb, a);
        else
            gather_block_wave<kMidGid, true, false>(A, gb, tb, a);
        const TwHalfRes<kMidGid> tw0{buf_rsrc(A.tw, (uint32_t)G.twoff[G.npass] * 8u), lds_tw, tb};
        static_for<0, Mid::V>([&](auto Uu) {
            hr_load_rows<kMidGid, decltype(Uu)::value>(r[decltype(Uu)::value], tw0);
        });
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
        const __amdgpu_buffer_rsrc_t rtw = buf_rsrc(twp, (uint32_t)G.twoff[G.npass] * 8u);
        const __amdgpu_buffer_rsrc_t rh = buf_rsrc(hp, (uint32_t)G.N * 8u);
        hr_transform<kMidGid>(
            tb, a, r, lds, TwHalfRes<kMidGid>{rtw, lds_tw, tb}, rh,
            [&](auto Uu, const float2(&v)[64]) {
                constexpr int u = decltype(Uu)::value;
                const int qu = fresh_v(qo);
                static_for<0, Mid::R0>([&](auto J) {
                    constexpr int rr = Mid::R0 * u + decltype(J)::value;
                    const int q = qu + G.TB * pass0_m<kMidGid>(rr);
                    if constexpr (REAL) {
                        buf_store_f32(v[rr].x, ry1, buf_off<4>(q));
                        buf_store_f32(v[rr].y, ry2, buf_off<4>(q));
                    } else {
                        buf_store(v[rr], ry, buf_off<8>(q));
                    }
                });
            },
            [&](auto Uu, float2(&v)[64]) {
                constexpr int u = decltype(Uu)::value;
                if (gn >= 0) {
                    if constexpr (REAL)
                        hr_gather_real<kMidGid, Mid::R0 * u, Mid::R0 * u + Mid::R0>(A, gn, tb, v);
                    else
                        gather_block_wave<kMidGid, true, false, Mid::R0 * u,
                                          Mid::R0 * u + Mid::R0>(A, gn, tb, v);
                }
            });
        if (i == A.nblk - 1)
            carry_state<kMidGid>(A.nsamples, Mm1, tb, ChanIn<REAL>(A, c), A.s0_old + c * Mm1,
                                 A.s0_new + c * Mm1);
        gb = gn;
    }
}

// H[(32 h + k) TB + tb] = DFT_N(taps)[bin] / N in the kernel's order: the
// forward half of the transform above, one workgroup.
__global__ __launch_bounds__(Mid::TB) void ols_mid_plan_taps_kernel(
    const float2 *__restrict__ taps, float2 *__restrict__ H, const float2 *__restrict__ tw) {
    constexpr Geo G = Mid::G;
    __shared__ float2 lds[Mid::HALF_SLOTS];
    const int tb = threadIdx.x;
    const TwTable<kMidGid> twt{tw, tb};
    float2 a[G.P];
    static_for<0, G.P>([&](auto Rr) {
        constexpr int rr = decltype(Rr)::value;
        a[rr] = taps[tb + G.TB * pass0_m<kMidGid>(rr)];
    });
    static_for<0, Mid::V>([&](auto Uu) {
        constexpr int u = decltype(Uu)::value;
        float2 r[Mid::NROWS];
        hr_load_rows<kMidGid, u>(r, twt);
        dft_at<Mid::R0, -1, Mid::R0 * u>(a);
        hr_pass0_twiddles<kMidGid, u, 1, Mid::HS, false>(a, r);
        hr_put0<kMidGid, u, 0>(tb, a, lds);
        hr_pass0_twiddles<kMidGid, u, Mid::HS, Mid::R0, false>(a, r);
    });
    constexpr float scale = 1.0f / G.N;
    static_for<0, 2>([&](auto Hh) {
        constexpr int h = decltype(Hh)::value;
        if constexpr (h == 1) {
            __syncthreads();
            static_for<0, Mid::V>([&](auto Uu) { hr_put0<kMidGid, decltype(Uu)::value, 1>(tb, a, lds); });
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
            H[(32 * h + k) * G.TB + tb] = make_float2(c[k].x * scale, c[k].y * scale);
        });
    });
}

int mid_geometry() { return kMidGid; }

int mid_max_groups(int device) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
        cus < 1)
        cus = 1;
    // the plan's workgroup count serves both variants: the smaller occupancy
    int per_cu_real = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, ols_mid_kernel<false>, Mid::TB,
                                                     0) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_real, ols_mid_kernel<true>, Mid::TB,
                                                     0) == hipSuccess &&
        per_cu_real >= 1 && per_cu_real < per_cu)
        per_cu = per_cu_real;
    return cus * per_cu;
}

hipError_t launch_mid(const FusedArgs &a, int max_groups, hipStream_t stream, bool real) {
    const int64_t units = a.nblk * a.nchan;
    if (units <= 0) return hipErrorInvalidConfiguration;
    int64_t grid = units;
    if (grid > max_groups) grid = max_groups & ~7;    // persistent, multiple of 8
    if (grid <= 0) grid = units < max_groups ? units : max_groups;
    if (real)
        hipLaunchKernelGGL(ols_mid_kernel<true>, dim3((unsigned)grid), dim3(Mid::TB), 0, stream, a);
    else
        hipLaunchKernelGGL(ols_mid_kernel<false>, dim3((unsigned)grid), dim3(Mid::TB), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_mid_plan_taps(const float2 *taps, float2 *H, const float2 *tw,
                                hipStream_t stream) {
    hipLaunchKernelGGL(ols_mid_plan_taps_kernel, dim3(1), dim3(Mid::TB), 0, stream, taps, H, tw);
    return hipGetLastError();
}

}  // namespace firols
