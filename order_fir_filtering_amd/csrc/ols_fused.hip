// LDS-resident overlap-save kernel: one N-point block per TB threads.
//
// Per block E_i (method page, claim 1): gather E_i = {D_(i-1), B_i} from
// the input, with the carried state S0 in front of the first block (step
// 3); forward N-point FFT, product with H, inverse FFT (step 4); drop the
// first M-1 points and store the L kept ones (step 5).  The block never
// leaves registers and LDS between the gather and the store.  The block
// that ends a channel also writes the channel's next state (the last M-1
// samples of {S0, x}) into the second state buffer, so no block reads
// memory another block of the same call writes.
#include <cmath>

#include "kernels.hpp"
#include "ols_phases.hpp"

namespace firols {

template <int LOGN>
struct FusedCfg {
    static constexpr Geo G = make_geo(LOGN);
    static constexpr int BPW = blocks_per_wg(LOGN);
    static constexpr int WG = G.TB * BPW;
    static constexpr int LDSN = G.npass > 1 ? G.lds_stride * BPW : 1;
};

// Forward passes with LDS exchanges between them.
template <int LOGN>
__device__ __forceinline__ void forward_all(int tb, float2 (&a)[make_geo(LOGN).P],
                                            float2 *lds, const float2 *__restrict__ tw) {
    constexpr Geo G = make_geo(LOGN);
    static_for<0, G.npass>([&](auto Sx) {
        constexpr int s = decltype(Sx)::value;
        if constexpr (s > 0) {
            __syncthreads();
            lds_put<LOGN, s - 1>(tb, a, lds);
            __syncthreads();
            lds_get<LOGN, s>(tb, a, lds);
        }
        fwd_pass<LOGN, s>(tb, a, tw);
    });
}

// Inverse passes in reverse order with LDS exchanges between them.
template <int LOGN>
__device__ __forceinline__ void inverse_all(int tb, float2 (&a)[make_geo(LOGN).P],
                                            float2 *lds, const float2 *__restrict__ tw) {
    constexpr Geo G = make_geo(LOGN);
    static_for<0, G.npass>([&](auto Ix) {
        constexpr int s = G.npass - 1 - decltype(Ix)::value;
        if constexpr (s < G.npass - 1) {
            __syncthreads();
            lds_put<LOGN, s + 1>(tb, a, lds);
            __syncthreads();
            lds_get<LOGN, s>(tb, a, lds);
        }
        inv_pass<LOGN, s>(tb, a, tw);
    });
}

template <int LOGN>
__global__ __launch_bounds__(FusedCfg<LOGN>::WG) void ols_fused_kernel(FusedArgs A) {
    using C = FusedCfg<LOGN>;
    constexpr Geo G = make_geo(LOGN);
    __shared__ float2 lds[C::LDSN];

    const int tid = threadIdx.x;
    const int sub = tid / G.TB;
    const int tb = tid - sub * G.TB;
    float2 *my = lds + sub * G.lds_stride;

    const int64_t total = A.nblk * A.nchan;
    const int64_t gb = (int64_t)blockIdx.x * C::BPW + sub;
    const bool active = gb < total;
    const int64_t c = active ? gb / A.nblk : 0;
    const int64_t i = active ? gb - c * A.nblk : 0;
    const int Mm1 = A.M - 1;
    const float2 *__restrict__ xc = A.x + c * A.stride;
    const float2 *__restrict__ sc = A.s0_old + c * Mm1;

    // Step 3: E_i[q] = xt[i L - (M-1) + q], xt = {S0, x, zeros}.
    float2 a[G.P];
    const int64_t g0 = i * A.L - Mm1;
    if (active && g0 >= 0 && g0 + G.N <= A.nsamples) {
        static_for<0, G.P>([&](auto Rr) {
            constexpr int r = decltype(Rr)::value;
            a[r] = xc[g0 + tb + G.TB * pass0_m<LOGN>(r)];
        });
    } else {
        static_for<0, G.P>([&](auto Rr) {
            constexpr int r = decltype(Rr)::value;
            const int64_t g = g0 + tb + G.TB * pass0_m<LOGN>(r);
            float2 v = make_float2(0.f, 0.f);
            if (active) {
                if (g < 0)
                    v = sc[Mm1 + g];
                else if (g < A.nsamples)
                    v = xc[g];
            }
            a[r] = v;
        });
    }

    // Step 4: F = FFT(E), I = F * H, R = IFFT(I) (1/N is folded into H).
    forward_all<LOGN>(tb, a, my, A.tw);
    mul_h<LOGN>(tb, a, A.H);
    inverse_all<LOGN>(tb, a, my, A.tw);

    if (!active) return;

    // Step 5: position q >= M-1 is output i L + q - (M-1).
    float2 *__restrict__ yc = A.y + c * A.stride;
    static_for<0, G.P>([&](auto Rr) {
        constexpr int r = decltype(Rr)::value;
        const int q = tb + G.TB * pass0_m<LOGN>(r);
        const int64_t o = g0 + q;
        if (q >= Mm1 && o < A.nsamples) yc[o] = a[r];
    });

    // State carry: the last M-1 samples of {S0, x} of this channel.
    if (i == A.nblk - 1) {
        float2 *__restrict__ sn = A.s0_new + c * Mm1;
        for (int r = tb; r < Mm1; r += G.TB) {
            const int64_t g = A.nsamples - Mm1 + r;
            sn[r] = g >= 0 ? xc[g] : sc[Mm1 + g];
        }
    }
}

// H[r * TB + tb] = DFT_N(taps)[bin] / N, in the order the fused kernel uses.
template <int LOGN>
__global__ __launch_bounds__(make_geo(LOGN).TB) void ols_plan_taps_kernel(
    const float2 *__restrict__ taps, float2 *__restrict__ H, const float2 *__restrict__ tw) {
    constexpr Geo G = make_geo(LOGN);
    __shared__ float2 lds[G.npass > 1 ? G.lds_stride : 1];
    const int tb = threadIdx.x;
    float2 a[G.P];
    static_for<0, G.P>([&](auto Rr) {
        constexpr int r = decltype(Rr)::value;
        a[r] = taps[tb + G.TB * pass0_m<LOGN>(r)];
    });
    forward_all<LOGN>(tb, a, lds, tw);
    constexpr float scale = 1.0f / G.N;
    static_for<0, G.P>([&](auto Rr) {
        constexpr int r = decltype(Rr)::value;
        H[r * G.TB + tb] = make_float2(a[r].x * scale, a[r].y * scale);
    });
}

__global__ __launch_bounds__(256) void copy_kernel(float2 *__restrict__ dst,
                                                   const float2 *__restrict__ src,
                                                   int64_t count) {
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; k < count; k += step)
        dst[k] = src ? src[k] : make_float2(0.f, 0.f);
}

template <int LOGN>
static hipError_t launch_fused_t(const FusedArgs &a, hipStream_t stream) {
    using C = FusedCfg<LOGN>;
    const int64_t total = a.nblk * a.nchan;
    const int64_t grid = (total + C::BPW - 1) / C::BPW;
    if (grid <= 0 || grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(ols_fused_kernel<LOGN>, dim3((unsigned)grid), dim3(C::WG), 0, stream, a);
    return hipGetLastError();
}

template <int LOGN>
static hipError_t launch_plan_t(const float2 *taps, float2 *H, const float2 *tw,
                                hipStream_t stream) {
    hipLaunchKernelGGL(ols_plan_taps_kernel<LOGN>, dim3(1), dim3(make_geo(LOGN).TB), 0, stream,
                       taps, H, tw);
    return hipGetLastError();
}

hipError_t launch_fused(int logn, const FusedArgs &a, hipStream_t stream) {
    switch (logn) {
        case 3: return launch_fused_t<3>(a, stream);
        case 4: return launch_fused_t<4>(a, stream);
        case 5: return launch_fused_t<5>(a, stream);
        case 6: return launch_fused_t<6>(a, stream);
        case 7: return launch_fused_t<7>(a, stream);
        case 8: return launch_fused_t<8>(a, stream);
        case 9: return launch_fused_t<9>(a, stream);
        case 10: return launch_fused_t<10>(a, stream);
        case 11: return launch_fused_t<11>(a, stream);
        case 12: return launch_fused_t<12>(a, stream);
        case 13: return launch_fused_t<13>(a, stream);
        case 14: return launch_fused_t<14>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_plan_taps(int logn, const float2 *taps, float2 *H, const float2 *tw,
                            hipStream_t stream) {
    switch (logn) {
        case 3: return launch_plan_t<3>(taps, H, tw, stream);
        case 4: return launch_plan_t<4>(taps, H, tw, stream);
        case 5: return launch_plan_t<5>(taps, H, tw, stream);
        case 6: return launch_plan_t<6>(taps, H, tw, stream);
        case 7: return launch_plan_t<7>(taps, H, tw, stream);
        case 8: return launch_plan_t<8>(taps, H, tw, stream);
        case 9: return launch_plan_t<9>(taps, H, tw, stream);
        case 10: return launch_plan_t<10>(taps, H, tw, stream);
        case 11: return launch_plan_t<11>(taps, H, tw, stream);
        case 12: return launch_plan_t<12>(taps, H, tw, stream);
        case 13: return launch_plan_t<13>(taps, H, tw, stream);
        case 14: return launch_plan_t<14>(taps, H, tw, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_copy(float2 *dst, const float2 *src, int64_t count, hipStream_t stream) {
    if (count <= 0) return hipSuccess;
    int64_t blocks = (count + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, dst, src, count);
    return hipGetLastError();
}

int twiddle_count(int logn) { return make_geo(logn).twoff[make_geo(logn).npass]; }

void build_twiddles(int logn, float2 *out) {
    const Geo g = make_geo(logn);
    for (int s = 0; s < g.npass; ++s) {
        const int R = g.R[s], S = g.S[s];
        const int64_t span = (int64_t)S * R;
        for (int k = 1; k < R; ++k) {
            for (int t = 0; t < S; ++t) {
                const int64_t e = ((int64_t)t * k) % span;
                const double ang = -2.0 * M_PI * (double)e / (double)span;
                out[g.twoff[s] + (k - 1) * S + t] =
                    make_float2((float)std::cos(ang), (float)std::sin(ang));
            }
        }
    }
}

void build_h_permutation(int logn, int64_t *perm) {
    const Geo g = make_geo(logn);
    for (int r = 0; r < g.P; ++r)
        for (int tb = 0; tb < g.TB; ++tb)
            perm[(int64_t)r * g.TB + tb] = bin_of_position(g, last_pass_position(g, tb, r));
}

}  // namespace firols
