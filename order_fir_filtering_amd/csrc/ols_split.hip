// Overlap-save for N = 65536: each block is split into two 32768-point
// sub-convolutions, the 32768-point half-resident transform (ols_big.hpp)
// runs each of them in one workgroup, and a combine kernel forms the
// outputs.
//
// With Ns = N / 2, n = q + j Ns and k = k0 + 2 k' (a decimation in
// frequency by two):
//   X[k0 + 2 k'] = DFT_Ns(a_k0)[k'],  a_k0[q] = W_N^{q k0} (E[q] + (-1)^k0 E[q + Ns])
//   c_k0 = IDFT_Ns(X_k0 * H_k0),      H_k0[k'] = H[k0 + 2 k']
//   y[q + j Ns] = c_0[q] + (-1)^j W_N^{-q} c_1[q]
// (method page, claim 1: gather E_i with the carried state in front,
// step 3; FFT, product with H and inverse FFT, step 4; the first M-1
// points dropped, step 5).  ols_split_sub_kernel runs one (block, k0)
// sub-convolution per workgroup at a time and writes c_k0 to a scratch
// buffer; ols_split_combine_kernel reads both halves and writes the L kept
// outputs.  Blocks go in chunks so the scratch stays small.
#include <cmath>
#include <vector>

#include "ols_big.hpp"

namespace firols {

namespace {

constexpr int kNs = kBig.N;        // points of a sub-transform
constexpr int kRT = 2;             // sub-transforms per block

// Work order of the sub-kernel: workgroup w always runs sub-problem k0 of
// the blocks of its team; the two members of a team (k0 = 0, 1) sit on one
// XCD (w % 8) and walk the same block sequence, so the second gather of a
// block reads it from that XCD's L2.  Each XCD takes one contiguous eighth
// of the blocks.
struct SplitOrder {
    int k0;
    int64_t first, step, end;   // blocks first, first + step, ... < end
};

__device__ __forceinline__ SplitOrder split_order(int w, int G, int64_t nblocks) {
    SplitOrder o;
    if (G % (8 * kRT) == 0) {
        const int m = w >> 3;
        const int per_xcd = (G >> 3) / kRT;
        const int64_t chunk = (nblocks + 7) >> 3;
        const int64_t lo = (int64_t)(w & 7) * chunk;
        o.k0 = m % kRT;
        o.first = lo + m / kRT;
        o.step = per_xcd;
        o.end = lo + chunk < nblocks ? lo + chunk : nblocks;
    } else {
        o.k0 = w % kRT;
        o.first = w / kRT;
        o.step = G / kRT;
        o.end = nblocks;
    }
    return o;
}

// a_k0 of one block into the pass-0 layout (register r <-> q = tb + TB m),
// reading E[q] and E[q + Ns] through load(j, TB m) and W_N^{q k0} from row
// k0 of the top twiddles (row 0 is all ones).  The second input and the
// twiddle go in groups of 8 points, the next group requested before the
// current one is used, so the registers in flight stay bounded.
template <class LOAD>
__device__ __forceinline__ void split_gather(float2 (&a)[64], int tb, int k0, const LOAD &load,
                                             __amdgpu_buffer_rsrc_t rtt) {
    const float sg = k0 ? -1.f : 1.f;
    static_for<0, 64>([&](auto Rr) {
        constexpr int r = decltype(Rr)::value;
        a[r] = load(0, kBig.TB * pass0_m<kBigGid>(r));
    });
    constexpr int G = 8;
    float2 e[2][G], w[2][G];
    auto issue = [&](auto Gx) {
        constexpr int g = decltype(Gx)::value;
        static_for<0, G>([&](auto Ii) {
            constexpr int i = decltype(Ii)::value;
            constexpr int off = kBig.TB * pass0_m<kBigGid>(g * G + i);
            e[g & 1][i] = load(1, off);
            w[g & 1][i] = buf_load_cached(rtt, (uint32_t)tb * 8u, (uint32_t)off * 8u);
        });
    };
    issue(ic<0>{});
    static_for<0, 64 / G>([&](auto Gx) {
        constexpr int g = decltype(Gx)::value;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (g + 1 < 64 / G) issue(ic<g + 1>{});
        __builtin_amdgcn_sched_barrier(0);
        static_for<0, G>([&](auto Ii) {
            constexpr int i = decltype(Ii)::value;
            constexpr int r = g * G + i;
            const float2 s = make_float2(fmaf(sg, e[g & 1][i].x, a[r].x),
                                         fmaf(sg, e[g & 1][i].y, a[r].y));
            a[r] = cmul(s, w[g & 1][i]);
        });
    });
    __builtin_amdgcn_sched_barrier(0);
}

}  // namespace

__global__ __launch_bounds__(kBig.TB) void ols_split_sub_kernel(SplitArgs A) {
    __shared__ float2 lds[kHalfSlots + kTw1];
    float2 *lds_tw = lds + kHalfSlots;
    const int tb = threadIdx.x;
    for (int e = tb; e < kTw1; e += kBig.TB) lds_tw[e] = A.tw[kBig.twoff[1] + e];
    // (the first barrier of the transform orders these writes before use)
    const SplitOrder o = split_order(blockIdx.x, gridDim.x, A.nchunk);
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
        const float2 *twp = A.tw, *hp = A.H, *ttp = A.tw_top;
        asm volatile("" : "+s"(twp), "+s"(hp), "+s"(ttp));
        const __amdgpu_buffer_rsrc_t rtw = buf_rsrc(twp, (uint32_t)kBig.twoff[kBig.npass] * 8u);
        const __amdgpu_buffer_rsrc_t rh = buf_rsrc(hp + (int64_t)k0 * kNs, (uint32_t)kNs * 8u);
        const __amdgpu_buffer_rsrc_t rtt = buf_rsrc(ttp + (int64_t)k0 * kNs, (uint32_t)kNs * 8u);
        const TwBig tw{rtw, lds_tw, tb};

        float2 a[64], w0[15], w1[15];
        if (g0 >= 0 && g0 + kRT * kNs <= A.nsamples) {
            const __amdgpu_buffer_rsrc_t rx = buf_rsrc(xc + g0, (uint32_t)(kRT * kNs) * 8u);
            split_gather(a, tb, k0, [&](int j, int off) {
                return buf_load(rx, (uint32_t)tb * 8u, (uint32_t)(off + j * kNs) * 8u);
            }, rtt);
        } else {
            // first blocks (state in front) and the partial last block: two
            // range-checked loads per point, one over the valid input and one
            // over the state; at most one is in range, the other reads zero
            const int64_t xs = g0 > 0 ? g0 : 0;
            int64_t xn = A.nsamples - xs;
            xn = xn < 0 ? 0 : (xn > kRT * kNs ? kRT * kNs : xn);
            const __amdgpu_buffer_rsrc_t rx = buf_rsrc(xc + xs, (uint32_t)xn * 8u);
            const __amdgpu_buffer_rsrc_t rs = buf_rsrc(sc, g0 < 0 ? (uint32_t)Mm1 * 8u : 0u);
            const int dx = (int)(g0 - xs) + tb;     // q + dx indexes x from xs
            const int ds = (int)(g0 + Mm1) + tb;    // q + ds indexes the state
            split_gather(a, tb, k0, [&](int j, int off) {
                const int q = off + j * kNs;
                const float2 u = buf_load(rx, (uint32_t)(q + dx) * 8u, 0);
                const float2 v = buf_load(rs, (uint32_t)(q + ds) * 8u, 0);
                return make_float2(u.x + v.x, u.y + v.y);
            }, rtt);
        }
        load_pass0_twiddles<0, 1>(w0, tw);
        load_pass0_twiddles<1, 1>(w1, tw);

        // c_k0 to the scratch buffer, read once by the combine kernel
        const __amdgpu_buffer_rsrc_t rsc =
            buf_rsrc(A.scratch + lb * (kRT * kNs) + (int64_t)k0 * kNs, (uint32_t)kNs * 8u);
        big_transform(
            tb, a, w0, w1, lds, tw, rh,
            [&](auto Uu, const float2(&v)[64]) {
                constexpr int u = decltype(Uu)::value;
                static_for<0, 32>([&](auto J) {
                    constexpr int r = 32 * u + decltype(J)::value;
                    buf_store_so(v[r], rsc, (uint32_t)tb * 8u,
                                 (uint32_t)(kBig.TB * pass0_m<kBigGid>(r)) * 8u);
                });
            },
            [&](auto, float2(&)[64]) {});

        if (k0 == 0 && i == A.nblk - 1)
            carry_state<kBigGid>(A.nsamples, Mm1, tb, xc, sc, A.s0_new + c * Mm1);
    }
}

// One thread per (block, q): y[q + j Ns] = c_0[q] + (-1)^j W_N^{-q} c_1[q].
__global__ __launch_bounds__(256) void ols_split_combine_kernel(SplitArgs A) {
    const int64_t total = A.nchunk * kNs;
    const int Mm1 = A.M - 1;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
         t += (int64_t)gridDim.x * blockDim.x) {
        const int64_t lb = t / kNs;
        const int q = (int)(t - lb * kNs);
        const int64_t gb = A.blk0 + lb;
        const int64_t c = gb / A.nblk;
        const int64_t i = gb - c * A.nblk;
        const float2 *__restrict__ in = A.scratch + lb * (kRT * kNs) + q;
        const float2 b0 = in[0];
        const float2 b1 = cmulc(in[kNs], A.tw_top[kNs + q]);
        float2 *__restrict__ yc = A.y + c * A.stride;
        const int64_t o0 = i * A.L - Mm1;     // output index of position 0
        if (q >= Mm1 && o0 + q < A.nsamples) nt_store(yc + o0 + q, cadd(b0, b1));
        if (q + kNs >= Mm1 && o0 + q + kNs < A.nsamples) nt_store(yc + o0 + q + kNs, csub(b0, b1));
    }
}

int split_radix(int logn) { return logn > kBigLogN ? 1 << (logn - kBig.logn) : 1; }

int split_sub_twiddle_count() { return twiddle_count(kBigGid); }

int64_t split_top_twiddle_count(int logn) {
    return split_radix(logn) > 1 ? (int64_t)split_radix(logn) * kNs : 0;
}

void build_split_twiddles(int logn, float2 *sub_tw, float2 *top_tw) {
    const int RT = split_radix(logn);
    const int64_t N = (int64_t)kNs * RT;
    build_twiddles(kBigGid, sub_tw);
    for (int k0 = 0; k0 < RT; ++k0)
        for (int q = 0; q < kNs; ++q) {
            const int64_t e = ((int64_t)q * k0) % N;
            const double ang = -2.0 * M_PI * (double)e / (double)N;
            top_tw[(int64_t)k0 * kNs + q] = make_float2((float)std::cos(ang), (float)std::sin(ang));
        }
}

void build_split_h_permutation(int logn, int64_t *perm) {
    const int RT = split_radix(logn);
    std::vector<int64_t> sub((size_t)kNs);
    build_h_permutation(kBigGid, sub.data());
    for (int k0 = 0; k0 < RT; ++k0)
        for (int i = 0; i < kNs; ++i) perm[(int64_t)k0 * kNs + i] = k0 + (int64_t)RT * sub[i];
}

int64_t split_block_elems(int logn) { return (int64_t)kNs * split_radix(logn); }

int split_max_groups(int device) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
        cus < 1)
        cus = 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, ols_split_sub_kernel, kBig.TB, 0) !=
            hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    return cus * per_cu;
}

hipError_t launch_split(int logn, const SplitArgs &a, int max_groups, hipStream_t stream) {
    if (a.nchunk <= 0 || split_radix(logn) != kRT) return hipErrorInvalidConfiguration;
    // a multiple of 2 workgroups (both k0 present); a multiple of 16 when
    // persistent, so the teams spread evenly over the XCDs
    const int64_t full = a.nchunk * kRT;
    const int64_t cap = (int64_t)(max_groups / (8 * kRT)) * (8 * kRT);
    int64_t grid = full;
    if (cap > 0 && full > cap) grid = cap;
    if (cap == 0 && full > max_groups) grid = max_groups / kRT > 0 ? (max_groups / kRT) * kRT : kRT;
    int64_t cgrid = (a.nchunk * kNs + 255) / 256;
    if (cgrid > 65536) cgrid = 65536;
    hipLaunchKernelGGL(ols_split_sub_kernel, dim3((unsigned)grid), dim3(kBig.TB), 0, stream, a);
    hipLaunchKernelGGL(ols_split_combine_kernel, dim3((unsigned)cgrid), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace firols
