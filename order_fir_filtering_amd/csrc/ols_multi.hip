// Overlap-save for N = 2^17 .. 2^20, more than one workgroup can hold: a
// four-step split N = RT * Ns of every block, with Ns = 32768 and
// RT = 4 .. 32, in three kernels per batch of blocks.
//
// With n = q + j Ns (q < Ns, j < RT) and k = k0 + RT k' (a decimation in
// frequency by RT):
//   top      a_k0[q] = W_N^{q k0} sum_j E[q + j Ns] W_RT^{j k0}
//   sub      c_k0 = IDFT_Ns(DFT_Ns(a_k0) * H_k0),  H_k0[k'] = H[k0 + RT k']
//   combine  R[q + j Ns] = sum_k0 W_RT^{-j k0} W_N^{-q k0} c_k0[q]
// which is R = IDFT_N(DFT_N(E) * H) of the method page, claim 1: E is the
// block {S0 or D_(i-1), B_i} (step 3), the transforms and the product
// with H are step 4, and of R the first M-1 points are dropped and the L
// others stored (step 5).  The top and combine kernels give each thread
// one q and its RT points in registers; the RT sub-convolutions of a
// block run on the 32768-point half-resident transform, one per
// workgroup, reading a_k0 from the scratch and writing c_k0 over it.  The
// scratch holds the batch's blocks ([unit][k0][q]), so a call runs in
// batches of as many blocks as it holds.
#include <cmath>

#include "ols_big.hpp"

namespace firols {

namespace {

constexpr int kNs = kBig.N;                // points of a sub-transform
constexpr int kQB = 256;                   // q values per workgroup of the top and combine kernels
constexpr int kQTiles = kNs / kQB;         // workgroups per block in those kernels
// Scratch of the plan: blocks of the batch times N values.
constexpr int64_t kScratchBytes = (int64_t)128 << 20;
// two floats as a clang vector, for the non-temporal store builtin
typedef float f32x2 __attribute__((ext_vector_type(2)));

// W_N^{q k0} with q = l + 256 h: the product of lo[k0][l] = W_N^{l k0}
// and hi[k0][h] = W_N^{256 h k0}, both from the plan's table (one table
// rounding each and one product).
template <int RT>
struct TopTw {
    const float2 *lo;   // this thread's column l of the [RT][256] part
    const float2 *hi;   // this workgroup's column h of the [RT][Ns / 256] part
    __device__ __forceinline__ TopTw(const float2 *t, int l, int h)
        : lo(t + l), hi(t + RT * kQB + h) {}
    __device__ __forceinline__ float2 operator()(int k0) const {
        return cmul(lo[k0 * kQB], hi[k0 * kQTiles]);
    }
};

// Sample n of block E (n in [0, N)) for a block that reaches past either
// end of the input: the state in front, zeros past the end.
template <class XC>
__device__ __forceinline__ float2 edge_sample(const XC &xc, const float2 *__restrict__ sc,
                                              int64_t g, int64_t nsamples, int Mm1) {
    if (g < 0) return sc[Mm1 + g];
    if (g < nsamples) return xc[g];
    return make_float2(0.f, 0.f);
}

// Sample g of real-pair channel c (rows 2c and 2c + 1 of a float32
// [2 nchan][stride] array are its real and imaginary parts).
struct RealPair {
    const float *__restrict__ x1;
    const float *__restrict__ x2;
    __device__ __forceinline__ float2 operator[](int64_t g) const {
        return make_float2(x1[g], x2[g]);
    }
};

template <bool REAL>
struct MultiIn;
template <>
struct MultiIn<false> {
    using T = const float2 *;
    static __device__ __forceinline__ T chan(const MultiArgs &A, int64_t c) {
        return A.x + c * A.stride;
    }
};
template <>
struct MultiIn<true> {
    using T = RealPair;
    static __device__ __forceinline__ T chan(const MultiArgs &A, int64_t c) {
        const float *x1 = (const float *)A.x + 2 * c * A.stride;
        return RealPair{x1, x1 + A.stride};
    }
};

// REAL: real-pair channels, read as RealPair and written as two float rows.
template <int LRT, bool REAL>
__global__ __launch_bounds__(kQB) void ols_multi_top_kernel(MultiArgs A) {
    constexpr int RT = 1 << LRT;
    const int tid = threadIdx.x;
    const int ul = blockIdx.x / kQTiles;      // unit within the batch
    const int qt = blockIdx.x - ul * kQTiles;
    const int q = qt * kQB + tid;
    const int64_t gb = A.u0 + ul;
    const int64_t c = gb / A.nblk;
    const int64_t i = gb - c * A.nblk;
    const int Mm1 = A.M - 1;
    const typename MultiIn<REAL>::T xc = MultiIn<REAL>::chan(A, c);
    const float2 *__restrict__ sc = A.s0_old + c * Mm1;
    const int64_t g0 = i * A.L - Mm1;

    float2 e[RT];
    if (g0 >= 0 && g0 + (int64_t)RT * kNs <= A.nsamples) {
        static_for<0, RT>([&](auto Jj) {
            constexpr int j = decltype(Jj)::value;
            e[j] = xc[g0 + q + (int64_t)j * kNs];
        });
    } else {
        static_for<0, RT>([&](auto Jj) {
            constexpr int j = decltype(Jj)::value;
            e[j] = edge_sample(xc, sc, g0 + q + (int64_t)j * kNs, A.nsamples, Mm1);
        });
    }
    dft<RT, -1>(e);
    float2 *__restrict__ out = A.scratch + (int64_t)ul * RT * kNs + q;
    const TopTw<RT> w(A.tw_top, tid, qt);
    out[0] = e[0];
    static_for<1, RT>([&](auto Kk) {
        constexpr int k0 = decltype(Kk)::value;
        out[(int64_t)k0 * kNs] = cmul(e[k0], w(k0));
    });

    // state carry: the channel's last block writes the last M-1 samples
    // of {S0, x}
    if (i == A.nblk - 1) {
        float2 *__restrict__ sn = A.s0_new + c * Mm1;
        for (int t = q; t < Mm1; t += kNs) {
            const int64_t g = A.nsamples - Mm1 + t;
            sn[t] = g >= 0 ? xc[g] : sc[Mm1 + g];
        }
    }
}

template <int LRT, bool REAL>
__global__ __launch_bounds__(kQB) void ols_multi_combine_kernel(MultiArgs A) {
    constexpr int RT = 1 << LRT;
    const int tid = threadIdx.x;
    const int ul = blockIdx.x / kQTiles;
    const int qt = blockIdx.x - ul * kQTiles;
    const int q = qt * kQB + tid;
    const int64_t gb = A.u0 + ul;
    const int64_t c = gb / A.nblk;
    const int64_t i = gb - c * A.nblk;
    const int Mm1 = A.M - 1;

    const float2 *__restrict__ in = A.scratch + (int64_t)ul * RT * kNs + q;
    float2 v[RT];
    static_for<0, RT>([&](auto Kk) {
        constexpr int k0 = decltype(Kk)::value;
        v[k0] = in[(int64_t)k0 * kNs];
    });
    const TopTw<RT> w(A.tw_top, tid, qt);
    static_for<1, RT>([&](auto Kk) {
        constexpr int k0 = decltype(Kk)::value;
        v[k0] = cmulc(v[k0], w(k0));
    });
    dft<RT, 1>(v);
    // R[q + j Ns] is output t = q + j Ns - (M-1) of the block when
    // 0 <= t < min(L, samples left)
    int64_t yn = A.nsamples - i * A.L;
    if (yn > A.L) yn = A.L;
    float2 *__restrict__ yb = A.y + c * A.stride + i * A.L;
    float *__restrict__ y1 = (float *)A.y + 2 * c * A.stride + i * A.L;
    static_for<0, RT>([&](auto Jj) {
        constexpr int j = decltype(Jj)::value;
        const int64_t t = (int64_t)q + (int64_t)j * kNs - Mm1;
        if (t >= 0 && t < yn) {
            if constexpr (REAL) {
                __builtin_nontemporal_store(v[j].x, y1 + t);
                __builtin_nontemporal_store(v[j].y, y1 + A.stride + t);
            } else {
                __builtin_nontemporal_store(__builtin_bit_cast(f32x2, v[j]), (f32x2 *)(yb + t));
            }
        }
    });
}

// The RT sub-convolutions of every block of the batch, one per workgroup
// iteration: a_k0 from the scratch in the pass-0 layout, the transform
// with H_k0, c_k0 back to the same positions.  Transform g is k0 = g / nu,
// unit g % nu, so the workgroups of one XCD (a contiguous range of g)
// mostly share one H_k0 in their L2.
__global__ __launch_bounds__(kBig.TB) void ols_multi_sub_kernel(MultiArgs A, int lrt) {
    __shared__ float2 lds[kHalfSlots + kTw1];
    float2 *lds_tw = lds + kHalfSlots;
    const int tb = threadIdx.x;
    for (int e = tb; e < kTw1; e += kBig.TB) lds_tw[e] = A.tw[kBig.twoff[1] + e];
    // (the first barrier of the transform orders these writes before use)
    const int64_t units = (int64_t)A.nu << lrt;
    auto slice = [&](int64_t g) {
        const int64_t k0 = g / A.nu;
        const int64_t u = g - k0 * A.nu;
        return buf_rsrc(A.scratch + ((u << lrt) + k0) * kNs, (uint32_t)kNs * 8u);
    };
    auto load = [&](auto R0, const __amdgpu_buffer_rsrc_t &rs, float2(&v)[64]) {
        constexpr int r0 = decltype(R0)::value;
        static_for<r0, r0 + 32>([&](auto Rr) {
            constexpr int r = decltype(Rr)::value;
            v[r] = buf_load_cached(rs, (uint32_t)tb * 8u,
                                   (uint32_t)(kBig.TB * pass0_m<kBigGid>(r)) * 8u);
        });
    };
    int64_t g = unit_of(units, blockIdx.x, gridDim.x, 0);
    float2 a[kBig.P];
    BigRows r;
    if (g >= 0) {
        const __amdgpu_buffer_rsrc_t rs = slice(g);
        load(ic<0>{}, rs, a);
        load(ic<32>{}, rs, a);
        const TwBig tw0{buf_rsrc(A.tw, (uint32_t)kBig.twoff[kBig.npass] * 8u), lds_tw, tb};
        load_big_rows(r, tw0);
    }
    for (int64_t it = 1; g >= 0; ++it) {
        const int64_t gn = unit_of(units, blockIdx.x, gridDim.x, it);
        // table pointers re-derived per transform so their loads stay in the loop
        const float2 *twp = A.tw, *hp = A.H;
        asm volatile("" : "+s"(twp), "+s"(hp));
        const int64_t k0 = g / A.nu;
        const __amdgpu_buffer_rsrc_t rs = slice(g);
        const __amdgpu_buffer_rsrc_t rn = slice(gn >= 0 ? gn : g);
        const __amdgpu_buffer_rsrc_t rtw = buf_rsrc(twp, (uint32_t)kBig.twoff[kBig.npass] * 8u);
        const __amdgpu_buffer_rsrc_t rh = buf_rsrc(hp + k0 * kNs, (uint32_t)kNs * 8u);
        big_transform(
            tb, a, r, lds, TwBig{rtw, lds_tw, tb}, rh,
            [&](auto Uu, const float2(&v)[64]) {
                constexpr int u = decltype(Uu)::value;
                static_for<0, 32>([&](auto J) {
                    constexpr int r = 32 * u + decltype(J)::value;
                    buf_store_cached(v[r], rs, (uint32_t)tb * 8u,
                                     (uint32_t)(kBig.TB * pass0_m<kBigGid>(r)) * 8u);
                });
            },
            [&](auto Uu, float2(&v)[64]) {
                if (gn >= 0) load(ic<32 * decltype(Uu)::value>{}, rn, v);
            });
        g = gn;
    }
}

template <int LRT, bool REAL>
hipError_t launch_batch(const MultiArgs &a, int max_groups, hipStream_t stream) {
    const dim3 gq((unsigned)a.nu * kQTiles);
    hipLaunchKernelGGL((ols_multi_top_kernel<LRT, REAL>), gq, dim3(kQB), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t units = (int64_t)a.nu << LRT;
    int64_t grid = units;
    if (grid > max_groups) grid = max_groups & ~7;    // persistent, multiple of 8
    if (grid <= 0) grid = units < max_groups ? units : max_groups;
    hipLaunchKernelGGL(ols_multi_sub_kernel, dim3((unsigned)grid), dim3(kBig.TB), 0, stream, a,
                       LRT);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((ols_multi_combine_kernel<LRT, REAL>), gq, dim3(kQB), 0, stream, a);
    return hipGetLastError();
}

template <bool REAL>
hipError_t launch_batch_r(int lrt, const MultiArgs &a, int max_groups, hipStream_t stream) {
    return lrt == 2   ? launch_batch<2, REAL>(a, max_groups, stream)
           : lrt == 3 ? launch_batch<3, REAL>(a, max_groups, stream)
           : lrt == 4 ? launch_batch<4, REAL>(a, max_groups, stream)
                      : launch_batch<5, REAL>(a, max_groups, stream);
}

}  // namespace

int64_t multi_top_twiddle_count(int logn) {
    const int64_t RT = split_radix(logn);
    return RT * (kQB + kQTiles);
}

void build_multi_top_twiddles(int logn, float2 *t) {
    const int RT = split_radix(logn);
    const int64_t N = (int64_t)1 << logn;
    auto w = [&](int64_t e) {
        const double ang = -2.0 * M_PI * (double)(e % N) / (double)N;
        return make_float2((float)std::cos(ang), (float)std::sin(ang));
    };
    for (int k0 = 0; k0 < RT; ++k0) {
        for (int l = 0; l < kQB; ++l) t[k0 * kQB + l] = w((int64_t)l * k0);
        for (int h = 0; h < kQTiles; ++h)
            t[RT * kQB + k0 * kQTiles + h] = w((int64_t)kQB * h * k0);
    }
}

int multi_batch_units(int logn) {
    const int64_t per_unit = ((int64_t)1 << logn) * (int64_t)sizeof(float2);
    const int64_t b = kScratchBytes / per_unit;
    return b > 0 ? (int)b : 1;
}

int multi_max_groups(int device) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
        cus < 1)
        cus = 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, ols_multi_sub_kernel, kBig.TB, 0) !=
            hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    return cus * per_cu;
}

// The call's units go through the scratch in batches of multi_batch_units;
// each batch is its top, sub and combine launches, in stream order.
hipError_t launch_multi(int logn, const MultiArgs &call, int max_groups, int64_t batch_units,
                        hipStream_t stream, bool real) {
    const int lrt = logn - kBig.logn;
    const int64_t units = call.nblk * call.nchan;
    if (lrt < 2 || lrt > 5 || units <= 0 || batch_units < 1) return hipErrorInvalidConfiguration;
    const int64_t batch = batch_units;
    for (int64_t u0 = 0; u0 < units; u0 += batch) {
        MultiArgs a = call;
        a.u0 = u0;
        a.nu = (int)(units - u0 < batch ? units - u0 : batch);
        hipError_t e = real ? launch_batch_r<true>(lrt, a, max_groups, stream)
                            : launch_batch_r<false>(lrt, a, max_groups, stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace firols
