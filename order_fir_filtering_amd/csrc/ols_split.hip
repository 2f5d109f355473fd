// Overlap-save for blocks larger than one CU holds (N = 32768, 65536).
//
// The N-point block transform (method page, claim 1, step 4) is split as
// N = RT * Ns with Ns = 16384, the largest transform one workgroup keeps in
// LDS.  With n = q + j Ns and k = k0 + RT k':
//
//   X[k0 + RT k'] = DFT_Ns(a_k0)[k'],
//   a_k0[q] = W_N^{q k0} * sum_j E[q + j Ns] W_RT^{j k0}            (gather)
//   y[q + j Ns] = sum_k0 W_RT^{-j k0} b_k0[q],
//   b_k0[q] = W_N^{-q k0} * IDFT_Ns(X_k0 * H_k0)[q]                 (combine)
//
// ols_split_sub_kernel runs one (block, k0) sub-convolution per workgroup:
// it gathers E (step 3, with the carried state), forms a_k0, runs the
// forward Ns-point FFT, multiplies by the bins k0 + RT k' of H, runs the
// inverse FFT and writes b_k0 to a scratch buffer.  ols_split_combine_kernel
// then forms the outputs, drops the first M-1 points of every block and
// stores the L kept ones (step 5).  The host runs a call in chunks of blocks
// so that the scratch buffer stays small enough to live in the last-level
// cache.
#include <cmath>
#include <vector>

#include "kernels.hpp"
#include "ols_block.hpp"

namespace firols {

namespace {

// Ns = 16384 points per workgroup: 512 threads x 32 points, radices 16, 32,
// 32 (two LDS exchanges per direction).  Pass 0's twiddles stay in 15
// registers per thread for the whole kernel (the second virtual thread's
// follow by a constant rotation); pass 1's table (992 values) is copied to
// LDS once.  No twiddle comes from global memory inside the loop.
constexpr int kSubGid = geo_id(14, 5);
constexpr Geo kSub = make_geo(kSubGid);
constexpr int kGroup = 16;                  // loads in flight per group

// v * W_RT^{e} with W_RT = exp(DIR * 2 pi i / RT), RT in {2, 4}, e constant.
template <int RT, int DIR, int E>
__device__ __forceinline__ float2 wrt(float2 v) {
    constexpr int e = ((E % RT) + RT) % RT;
    return rot16<DIR * e * (16 / RT)>(v);
}

// a_k0 of sub-problem k0 for the registers of thread tb:
//   RT = 2:  a = e0 + s e1,
//   RT = 4:  a = (e0 + s e2) + (-i)^k0 (e1 + s e3),   s = (-1)^k0,
// (the k0-th output of a radix-RT DFT over e_j = E[q + j Ns]), then times
// W_N^{q k0}.  k0 is a runtime value uniform over the workgroup, so one code
// path serves every k0.  Points go kGather at a time, with scheduling
// barriers, so at most RT * kGather loads are in flight.
constexpr int kGather = 8;
template <int RT, class LOAD>
__device__ __forceinline__ void split_gather(float2 (&a)[kSub.P], int tb, int k0,
                                             const LOAD &load,
                                             const float2 *__restrict__ tw_top) {
    static_assert(RT == 2 || RT == 4, "split radix");
    const float sg = (k0 & 1) ? -1.f : 1.f;
    // (-i)^k0 = (ca, sa): k0 = 0: (1, 0), 1: (0, -1), 2: (-1, 0), 3: (0, 1)
    const float ca = (k0 & 1) ? 0.f : ((k0 & 2) ? -1.f : 1.f);
    const float sa = (k0 & 1) ? ((k0 & 2) ? 1.f : -1.f) : 0.f;
    static_for<0, kSub.P / kGather>([&](auto Gx) {
        constexpr int g = decltype(Gx)::value;
        __builtin_amdgcn_sched_barrier(0);
        float2 e[RT][kGather];
        static_for<0, kGather>([&](auto Rr) {
            constexpr int r = g * kGather + decltype(Rr)::value;
            const int q = tb + kSub.TB * pass0_m<kSubGid>(r);
            static_for<0, RT>([&](auto J) {
                e[decltype(J)::value][decltype(Rr)::value] = load(q + decltype(J)::value * kSub.N);
            });
        });
        static_for<0, kGather>([&](auto Rr) {
            constexpr int r = g * kGather + decltype(Rr)::value;
            constexpr int i = decltype(Rr)::value;
            if constexpr (RT == 2) {
                a[r] = make_float2(fmaf(sg, e[1][i].x, e[0][i].x), fmaf(sg, e[1][i].y, e[0][i].y));
            } else {
                const float2 u = make_float2(fmaf(sg, e[2][i].x, e[0][i].x),
                                             fmaf(sg, e[2][i].y, e[0][i].y));
                const float2 v = make_float2(fmaf(sg, e[3][i].x, e[1][i].x),
                                             fmaf(sg, e[3][i].y, e[1][i].y));
                a[r] = make_float2(fmaf(ca, v.x, fmaf(-sa, v.y, u.x)),
                                   fmaf(ca, v.y, fmaf(sa, v.x, u.y)));
            }
        });
    });
    if (k0 > 0) {
        const float2 *__restrict__ tt = tw_top + (int64_t)(k0 - 1) * kSub.N + tb;
        static_for<0, kSub.P / kGather>([&](auto Gx) {
            constexpr int g = decltype(Gx)::value;
            __builtin_amdgcn_sched_barrier(0);
            static_for<0, kGather>([&](auto Rr) {
                constexpr int r = g * kGather + decltype(Rr)::value;
                a[r] = cmul(a[r], tt[kSub.TB * pass0_m<kSubGid>(r)]);
            });
        });
    }
    __builtin_amdgcn_sched_barrier(0);
}

// Product with the bins k0 + RT k' of H (sub-kernel order), in groups.
__device__ __forceinline__ void split_mul_h(float2 (&a)[kSub.P], int tb,
                                            const float2 *__restrict__ H) {
    static_for<0, kSub.P / kGroup>([&](auto Gx) {
        constexpr int g = decltype(Gx)::value;
        __builtin_amdgcn_sched_barrier(0);
        static_for<0, kGroup>([&](auto Rr) {
            constexpr int r = g * kGroup + decltype(Rr)::value;
            a[r] = cmul(a[r], H[r * kSub.TB + tb]);
        });
    });
    __builtin_amdgcn_sched_barrier(0);
}

// Work order of the sub-kernel: workgroup w always runs sub-problem k0 of
// the blocks of its team; the RT members of a team (k0 = 0 .. RT-1) sit on
// one XCD (w % 8) and walk the same block sequence, so the RT gathers of a
// block read it once from HBM and then from that XCD's L2.  Each XCD takes
// one contiguous eighth of the blocks.
struct SplitOrder {
    int k0;
    int64_t first, step, end;   // blocks first, first + step, ... < end
};

template <int RT>
__device__ __forceinline__ SplitOrder split_order(int w, int G, int64_t nblocks) {
    SplitOrder o;
    if (G % (8 * RT) == 0) {
        const int m = w >> 3;
        const int per_xcd = (G >> 3) / RT;
        const int64_t chunk = (nblocks + 7) >> 3;
        const int64_t lo = (int64_t)(w & 7) * chunk;
        o.k0 = m % RT;
        o.first = lo + m / RT;
        o.step = per_xcd;
        o.end = lo + chunk < nblocks ? lo + chunk : nblocks;
    } else {
        o.k0 = w % RT;
        o.first = w / RT;
        o.step = G / RT;
        o.end = nblocks;
    }
    return o;
}

// The persistent loop of a workgroup (sub-problem o.k0 of its team's blocks).
template <int RT>
__device__ __forceinline__ void split_sub_loop(const SplitArgs &A, const SplitOrder &o,
                                               float2 *lds, const TwRegLds<kSubGid> &tw) {
    constexpr int N = kSub.N * RT;
    const int tb = threadIdx.x;
    const int Mm1 = A.M - 1;
    const int k0 = o.k0;
    for (int64_t lb = o.first; lb < o.end; lb += o.step) {
        const int64_t gb = A.blk0 + lb;
        const int64_t c = gb / A.nblk;
        const int64_t i = gb - c * A.nblk;
        const float2 *__restrict__ xc = A.x + c * A.stride;
        const float2 *__restrict__ sc = A.s0_old + c * Mm1;
        const int64_t g0 = i * A.L - Mm1;
        // table pointers re-derived per block so their loads stay in the loop
        const float2 *hp = A.H, *ttp = A.tw_top;
        asm volatile("" : "+s"(hp), "+s"(ttp));

        float2 a[kSub.P];
        if (g0 >= 0 && g0 + N <= A.nsamples) {
            const float2 *__restrict__ xb = xc + g0;
            split_gather<RT>(a, tb, k0, [&](int q) { return xb[q]; }, ttp);
        } else {
            // first blocks (state in front) and the partial last block: two
            // range-checked loads per point, one over the valid input and one
            // over the state; at most one is in range, the other reads zero.
            const int64_t xs = g0 > 0 ? g0 : 0;
            int64_t xn = A.nsamples - xs;
            xn = xn < 0 ? 0 : (xn > N ? N : xn);
            const __amdgpu_buffer_rsrc_t rx = buf_rsrc(xc + xs, (uint32_t)xn * 8u);
            const __amdgpu_buffer_rsrc_t rs = buf_rsrc(sc, g0 < 0 ? (uint32_t)Mm1 * 8u : 0u);
            const int dx = (int)(g0 - xs);          // <= 0
            const int ds = (int)(g0 + Mm1);         // >= 0
            split_gather<RT>(a, tb, k0, [&](int q) {
                const float2 u = buf_load(rx, (uint32_t)(q + dx) * 8u, 0);
                const float2 v = buf_load(rs, (uint32_t)(q + ds) * 8u, 0);
                return make_float2(u.x + v.x, u.y + v.y);
            }, ttp);
        }

        forward_all<kSubGid>(tb, a, lds, tw);
        split_mul_h(a, tb, hp + (int64_t)k0 * kSub.N);
        inverse_all<kSubGid>(tb, a, lds, tw);

        float2 *__restrict__ out = A.scratch + lb * N + (int64_t)k0 * kSub.N;
        const float2 *__restrict__ tt = ttp + (int64_t)(k0 > 0 ? k0 - 1 : 0) * kSub.N;
        static_for<0, kSub.P / kGroup>([&](auto Gx) {
            constexpr int g = decltype(Gx)::value;
            __builtin_amdgcn_sched_barrier(0);
            static_for<0, kGroup>([&](auto Rr) {
                constexpr int r = g * kGroup + decltype(Rr)::value;
                const int q = tb + kSub.TB * pass0_m<kSubGid>(r);
                float2 v = a[r];
                if (k0 > 0) v = cmulc(v, tt[q]);
                nt_store(out + q, v);   // read once by the combine kernel
            });
        });

        if (k0 == 0 && i == A.nblk - 1)
            carry_state<kSubGid>(A.nsamples, Mm1, tb, xc, sc, A.s0_new + c * Mm1);
    }
}

}  // namespace

template <int RT>
__global__ __launch_bounds__(kSub.TB) void ols_split_sub_kernel(SplitArgs A) {
    // exchange buffer, then the pass-1 twiddle table
    __shared__ float2 lds[kSub.lds_stride + TwRegLds<kSubGid>::lds_count];
    const SplitOrder o = split_order<RT>(blockIdx.x, gridDim.x, A.nchunk);
    float2 *lds_tw = lds + kSub.lds_stride;
    for (int e = threadIdx.x; e < TwRegLds<kSubGid>::lds_count; e += kSub.TB)
        lds_tw[e] = A.tw[kSub.twoff[1] + e];
    __syncthreads();
    TwRegLds<kSubGid> tw;
    tw.load(A.tw, lds_tw, threadIdx.x);
    split_sub_loop<RT>(A, o, lds, tw);
}

// One thread per (block, q): y[q + j Ns] = sum_k0 W_RT^{-j k0} b_k0[q].
template <int RT>
__global__ __launch_bounds__(256) void ols_split_combine_kernel(SplitArgs A) {
    constexpr int N = kSub.N * RT;
    const int64_t total = A.nchunk * kSub.N;
    const int Mm1 = A.M - 1;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t lb = t / kSub.N;
        const int q = (int)(t - lb * kSub.N);
        const int64_t gb = A.blk0 + lb;
        const int64_t c = gb / A.nblk;
        const int64_t i = gb - c * A.nblk;
        const float2 *__restrict__ in = A.scratch + lb * N + q;
        float2 b[RT];
        static_for<0, RT>([&](auto K) { b[decltype(K)::value] = in[decltype(K)::value * kSub.N]; });
        float2 *__restrict__ yc = A.y + c * A.stride;
        const int64_t o0 = i * A.L - Mm1;     // output index of position 0
        static_for<0, RT>([&](auto J) {
            constexpr int j = decltype(J)::value;
            float2 s = b[0];
            static_for<1, RT>([&](auto K) {
                constexpr int k = decltype(K)::value;
                s = cadd(s, wrt<RT, 1, j * k>(b[k]));
            });
            const int n = q + j * kSub.N;
            const int64_t o = o0 + n;
            if (n >= Mm1 && o < A.nsamples) nt_store(yc + o, s);
        });
    }
}

// H[k0 Ns + r TB + tb] = DFT_N(taps)[k0 + RT * bin(tb, r)] / N: one
// workgroup per k0 runs the gather and the forward sub-transform.
template <int RT>
__global__ __launch_bounds__(kSub.TB) void ols_split_plan_taps_kernel(
    const float2 *__restrict__ taps, float2 *__restrict__ H, const float2 *__restrict__ tw,
    const float2 *__restrict__ tw_top) {
    __shared__ float2 lds[kSub.lds_stride];
    const int tb = threadIdx.x;
    const int k0 = blockIdx.x;
    float2 a[kSub.P];
    split_gather<RT>(a, tb, k0, [&](int q) { return taps[q]; }, tw_top);
    forward_all<kSubGid>(tb, a, lds, TwTable<kSubGid>{tw, tb});
    constexpr float scale = 1.0f / (kSub.N * RT);
    static_for<0, kSub.P>([&](auto Rr) {
        constexpr int r = decltype(Rr)::value;
        H[(int64_t)k0 * kSub.N + r * kSub.TB + tb] = make_float2(a[r].x * scale, a[r].y * scale);
    });
}

int split_radix(int logn) { return logn > kBigLogN ? 1 << (logn - kSub.logn) : 1; }

int split_sub_twiddle_count() { return twiddle_count(kSubGid); }

void build_split_twiddles(int logn, float2 *sub_tw, float2 *top_tw) {
    const int RT = split_radix(logn);
    const int64_t N = (int64_t)kSub.N * RT;
    build_twiddles(kSubGid, sub_tw);
    for (int k0 = 1; k0 < RT; ++k0)
        for (int q = 0; q < kSub.N; ++q) {
            const int64_t e = ((int64_t)q * k0) % N;
            const double ang = -2.0 * M_PI * (double)e / (double)N;
            top_tw[(int64_t)(k0 - 1) * kSub.N + q] =
                make_float2((float)std::cos(ang), (float)std::sin(ang));
        }
}

void build_split_h_permutation(int logn, int64_t *perm) {
    const int RT = split_radix(logn);
    std::vector<int64_t> sub((size_t)kSub.N);
    build_h_permutation(kSubGid, sub.data());
    for (int k0 = 0; k0 < RT; ++k0)
        for (int i = 0; i < kSub.N; ++i) perm[(int64_t)k0 * kSub.N + i] = k0 + (int64_t)RT * sub[i];
}

int64_t split_block_elems(int logn) { return (int64_t)kSub.N * split_radix(logn); }

int split_max_groups(int device) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
        cus < 1)
        cus = 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, ols_split_sub_kernel<4>, kSub.TB,
                                                     0) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    return cus * per_cu;
}

hipError_t launch_split(int logn, const SplitArgs &a, int max_groups, hipStream_t stream) {
    const int RT = split_radix(logn);
    if (a.nchunk <= 0 || RT < 2) return hipErrorInvalidConfiguration;
    // a multiple of RT workgroups (every k0 present); a multiple of 8 * RT
    // when persistent, so the teams spread evenly over the XCDs
    const int64_t full = a.nchunk * RT;
    const int64_t cap = (int64_t)(max_groups / (8 * RT)) * (8 * RT);
    int64_t grid = full;
    if (cap > 0 && full > cap) grid = cap;
    if (cap == 0 && full > max_groups) grid = max_groups / RT > 0 ? (max_groups / RT) * RT : RT;
    int64_t cgrid = (a.nchunk * kSub.N + 255) / 256;
    if (cgrid > 65536) cgrid = 65536;
    if (RT == 2) {
        hipLaunchKernelGGL(ols_split_sub_kernel<2>, dim3((unsigned)grid), dim3(kSub.TB), 0,
                           stream, a);
        hipLaunchKernelGGL(ols_split_combine_kernel<2>, dim3((unsigned)cgrid), dim3(256), 0,
                           stream, a);
    } else if (RT == 4) {
        hipLaunchKernelGGL(ols_split_sub_kernel<4>, dim3((unsigned)grid), dim3(kSub.TB), 0,
                           stream, a);
        hipLaunchKernelGGL(ols_split_combine_kernel<4>, dim3((unsigned)cgrid), dim3(256), 0,
                           stream, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_split_plan_taps(int logn, const float2 *taps, float2 *H, const float2 *tw,
                                  const float2 *tw_top, hipStream_t stream) {
    const int RT = split_radix(logn);
    if (RT == 2)
        hipLaunchKernelGGL(ols_split_plan_taps_kernel<2>, dim3(2), dim3(kSub.TB), 0, stream, taps,
                           H, tw, tw_top);
    else if (RT == 4)
        hipLaunchKernelGGL(ols_split_plan_taps_kernel<4>, dim3(4), dim3(kSub.TB), 0, stream, taps,
                           H, tw, tw_top);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace firols
