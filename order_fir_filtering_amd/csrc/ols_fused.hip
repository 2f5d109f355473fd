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
#include "ols_block.hpp"

namespace firols {

template <int GID>
struct FusedCfg {
    static constexpr Geo G = make_geo(GID);
    static constexpr int BPW = blocks_per_wg(GID);
    static constexpr int WG = G.TB * BPW;
    static constexpr int LDSN = G.npass > 1 ? G.lds_stride * BPW : 1;
    // Twiddles and H stay in registers for the whole kernel when the VGPR
    // budget allows it (the workgroup runs many blocks, and a thread always
    // holds the same positions of each block).
    static constexpr bool REGS = G.logn <= 12;
    // Buffer-descriptor I/O needs whole waves per block (N >= 1024); smaller
    // blocks share a wave and use pointer I/O.  (N = 16384 has a kernel of
    // its own, ols_mid.hip.)
    static constexpr bool WAVE_IO = G.TB >= 64 && G.TB < 1024;
    static_assert(WAVE_IO || REGS, "the fused kernel covers N <= 8192");
    // At N = 8192 one block takes 66 KB of LDS and 8 waves, so two
    // workgroups fit a CU if a thread keeps to 128 VGPRs (4 waves per SIMD):
    // the second workgroup's gather and store then overlap the first one's
    // transform.  Measured with one long call at M = 2049: 94 GS/s with one
    // workgroup per CU (158 VGPRs), 131 GS/s with two (128 VGPRs, some
    // spilled to scratch).
    static constexpr int MIN_WAVES_PER_SIMD = G.logn == 13 ? 4 : 1;
};

// One block: gather (step 3), FFT / product / inverse FFT (step 4), store
// of the kept points (step 5), and the state carry of the channel's last
// block.  Inactive threads (padding sub-blocks) take part in the barriers.
// This form serves blocks smaller than a wavefront (several blocks share a
// wave), with plain pointer accesses.
template <int GID, bool REAL, class TW, class HP>
__device__ __forceinline__ void filter_block(const FusedArgs &A, int64_t gb, bool active, int tb,
                                             float2 *my, const TW &tw, const HP &hp) {
    constexpr Geo G = make_geo(GID);
    const int64_t c = active ? gb / A.nblk : 0;
    const int64_t i = active ? gb - c * A.nblk : 0;
    const int Mm1 = A.M - 1;
    const ChanIn<REAL> xc(A, c);
    const float2 *__restrict__ sc = A.s0_old + c * Mm1;

    // E_i[q] = xt[i L - (M-1) + q], xt = {S0, x, zeros}.
    float2 a[G.P];
    const int64_t g0 = i * A.L - Mm1;
    if (active && g0 >= 0 && g0 + G.N <= A.nsamples) {
        static_for<0, G.P>([&](auto Rr) {
            constexpr int r = decltype(Rr)::value;
            a[r] = xc[g0 + tb + G.TB * pass0_m<GID>(r)];
        });
    } else {
        static_for<0, G.P>([&](auto Rr) {
            constexpr int r = decltype(Rr)::value;
            const int64_t g = g0 + tb + G.TB * pass0_m<GID>(r);
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

    // F = FFT(E), I = F * H, R = IFFT(I) (1/N is folded into H).
    forward_all<GID>(tb, a, my, tw);
    mul_h<GID>(a, hp);
    inverse_all<GID>(tb, a, my, tw);

    if (!active) return;

    // Position q >= M-1 is output i L + q - (M-1).
    const int64_t lim = A.nsamples - g0 - tb;   // q - tb must stay below this
    if constexpr (REAL) {
        // the real part to row 2c, the imaginary part to row 2c + 1
        float *__restrict__ y1 = (float *)A.y + 2 * c * A.stride + g0 + tb;
        float *__restrict__ y2 = y1 + A.stride;
        static_for<0, G.P>([&](auto Rr) {
            constexpr int r = decltype(Rr)::value;
            constexpr int off = G.TB * pass0_m<GID>(r);
            if (tb + off >= Mm1 && off < lim) {
                y1[off] = a[r].x;
                y2[off] = a[r].y;
            }
        });
    } else {
        float2 *__restrict__ yb = A.y + c * A.stride + g0 + tb;
        static_for<0, G.P>([&](auto Rr) {
            constexpr int r = decltype(Rr)::value;
            constexpr int off = G.TB * pass0_m<GID>(r);
            if (tb + off >= Mm1 && off < lim) yb[off] = a[r];
        });
    }

    if (i == A.nblk - 1) carry_state<GID>(A.nsamples, Mm1, tb, xc, sc, A.s0_new + c * Mm1);
}

template <int GID, bool REAL, class TW, class HP>
__device__ __forceinline__ void process_block_wave(const FusedArgs &A, int64_t gb, int tb,
                                                   float2 (&a)[make_geo(GID).P], float2 *my,
                                                   const TW &tw, const HP &hp) {
    forward_all<GID>(tb, a, my, tw);
    mul_h<GID>(a, hp);
    inverse_all<GID>(tb, a, my, tw);

    store_block_wave<GID, REAL>(A, gb, tb, a);
}

// REAL: each channel is a pair of real float32 rows (see ChanIn).
template <int GID, bool REAL>
__global__ __launch_bounds__(FusedCfg<GID>::WG, FusedCfg<GID>::MIN_WAVES_PER_SIMD) void ols_fused_kernel(
    FusedArgs A) {
    using C = FusedCfg<GID>;
    constexpr Geo G = make_geo(GID);
    __shared__ float2 lds[C::LDSN];

    const int tid = threadIdx.x;
    // a block spans whole waves when TB >= 64: make that uniformity visible
    const int sub = C::WAVE_IO ? __builtin_amdgcn_readfirstlane(tid / G.TB) : tid / G.TB;
    const int tb = tid - sub * G.TB;
    float2 *my = lds + sub * G.lds_stride;
    const int64_t total = A.nblk * A.nchan;
    const int64_t units = (total + C::BPW - 1) / C::BPW;

    auto run = [&](const auto &tw, const auto &hp) {
        for (int64_t it = 0;; ++it) {
            const int64_t unit = unit_of(units, blockIdx.x, gridDim.x, it);
            if (unit < 0) break;
            const int64_t gb = unit * C::BPW + sub;
            filter_block<GID, REAL>(A, gb, gb < total, tb, my, tw, hp);
        }
    };
    if constexpr (C::WAVE_IO && C::REGS) {
        // the first block's input is requested before the register-held
        // twiddles and H, so the first pass only waits for its own data
        float2 a[G.P];
        int64_t unit = unit_of(units, blockIdx.x, gridDim.x, 0);
        if (unit >= 0) gather_block_wave<GID, false, true, 0, G.P, REAL>(A, unit * C::BPW + sub, tb, a);
        TwRegs<GID> tw;
        tw.load(A.tw, tb);
        HRegs<GID> hp;
        hp.load(A.H, tb);
        if (units <= (int64_t)gridDim.x) {
            // one block per workgroup: nothing to request ahead
            if (unit >= 0) process_block_wave<GID, REAL>(A, unit * C::BPW + sub, tb, a, my, tw, hp);
            return;
        }
        // several blocks per workgroup: the next block's input is requested
        // into a second register set before this block's transform, so its
        // loads are in flight while the transform runs (a and b alternate;
        // the transform itself issues no memory loads).  Measured on 1024
        // channels at N = 1024: 290 -> 303 GS/s; one long call at N = 2048:
        // 245 -> 268 GS/s.  These loads take the default cache policy: the
        // M-1 samples a block shares with the next one are then found in L2
        // more often when a neighbouring wave reads them (1024 channels at
        // N = 1024: 306 -> 315 GS/s against the non-temporal policy, which
        // the one-block-per-workgroup case keeps).
        float2 b[G.P];
        for (int64_t it = 1; unit >= 0; it += 2) {
            const int64_t u1 = unit_of(units, blockIdx.x, gridDim.x, it);
            if (u1 >= 0) gather_block_wave<GID, false, false, 0, G.P, REAL>(A, u1 * C::BPW + sub, tb, b);
            process_block_wave<GID, REAL>(A, unit * C::BPW + sub, tb, a, my, tw, hp);
            if (u1 < 0) break;
            const int64_t u2 = unit_of(units, blockIdx.x, gridDim.x, it + 1);
            if (u2 >= 0) gather_block_wave<GID, false, false, 0, G.P, REAL>(A, u2 * C::BPW + sub, tb, a);
            process_block_wave<GID, REAL>(A, u1 * C::BPW + sub, tb, b, my, tw, hp);
            unit = u2;
        }
    } else if constexpr (C::WAVE_IO) {
        for (int64_t it = 0;; ++it) {
            const int64_t unit = unit_of(units, blockIdx.x, gridDim.x, it);
            if (unit < 0) break;
            const float2 *twp = A.tw;
            const float2 *hpp = A.H;
            asm volatile("" : "+s"(twp), "+s"(hpp));
            const int64_t gb = unit * C::BPW + sub;
            float2 a[G.P];
            gather_block_wave<GID, false, true, 0, G.P, REAL>(A, gb, tb, a);
            process_block_wave<GID, REAL>(A, gb, tb, a, my, TwTable<GID>{twp, tb}, HTable<GID>{hpp, tb});
        }
    } else {
        TwRegs<GID> tw;
        tw.load(A.tw, tb);
        HRegs<GID> hp;
        hp.load(A.H, tb);
        run(tw, hp);
    }
}

// H[r * TB + tb] = DFT_N(taps)[bin] / N, in the order the fused kernel uses.
template <int GID>
__global__ __launch_bounds__(make_geo(GID).TB) void ols_plan_taps_kernel(
    const float2 *__restrict__ taps, float2 *__restrict__ H, const float2 *__restrict__ tw) {
    constexpr Geo G = make_geo(GID);
    __shared__ float2 lds[G.npass > 1 ? G.lds_stride : 1];
    const int tb = threadIdx.x;
    float2 a[G.P];
    static_for<0, G.P>([&](auto Rr) {
        constexpr int r = decltype(Rr)::value;
        a[r] = taps[tb + G.TB * pass0_m<GID>(r)];
    });
    forward_all<GID>(tb, a, lds, TwTable<GID>{tw, tb});
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

// Geometry of the fused kernel for each transform size (geometry.hpp).
constexpr int fused_gid(int logn) { return logn; }

int fused_geometry(int logn) { return fused_gid(logn); }

template <int GID>
static hipError_t launch_fused_t(const FusedArgs &a, int max_groups, hipStream_t stream,
                                 bool real) {
    using C = FusedCfg<GID>;
    const int64_t total = a.nblk * a.nchan;
    const int64_t units = (total + C::BPW - 1) / C::BPW;
    if (units <= 0) return hipErrorInvalidConfiguration;
    int64_t grid = units;
    if (grid > max_groups) grid = max_groups & ~7;    // persistent, multiple of 8
    if (grid <= 0) grid = units < max_groups ? units : max_groups;
    if (real)
        hipLaunchKernelGGL((ols_fused_kernel<GID, true>), dim3((unsigned)grid), dim3(C::WG), 0,
                           stream, a);
    else
        hipLaunchKernelGGL((ols_fused_kernel<GID, false>), dim3((unsigned)grid), dim3(C::WG), 0,
                           stream, a);
    return hipGetLastError();
}

template <int GID>
static hipError_t launch_plan_t(const float2 *taps, float2 *H, const float2 *tw,
                                hipStream_t stream) {
    hipLaunchKernelGGL(ols_plan_taps_kernel<GID>, dim3(1), dim3(make_geo(GID).TB), 0, stream,
                       taps, H, tw);
    return hipGetLastError();
}

hipError_t launch_fused(int logn, const FusedArgs &a, int max_groups, hipStream_t stream,
                        bool real) {
    switch (logn) {
        case 3: return launch_fused_t<fused_gid(3)>(a, max_groups, stream, real);
        case 4: return launch_fused_t<fused_gid(4)>(a, max_groups, stream, real);
        case 5: return launch_fused_t<fused_gid(5)>(a, max_groups, stream, real);
        case 6: return launch_fused_t<fused_gid(6)>(a, max_groups, stream, real);
        case 7: return launch_fused_t<fused_gid(7)>(a, max_groups, stream, real);
        case 8: return launch_fused_t<fused_gid(8)>(a, max_groups, stream, real);
        case 9: return launch_fused_t<fused_gid(9)>(a, max_groups, stream, real);
        case 10: return launch_fused_t<fused_gid(10)>(a, max_groups, stream, real);
        case 11: return launch_fused_t<fused_gid(11)>(a, max_groups, stream, real);
        case 12: return launch_fused_t<fused_gid(12)>(a, max_groups, stream, real);
        case 13: return launch_fused_t<fused_gid(13)>(a, max_groups, stream, real);
        default: return hipErrorInvalidValue;
    }
}

// Resident workgroups per CU of both variants (complex and real-pair
// channels), the smaller of the two.
template <int GID>
static int max_groups_t(int cus) {
    int pc = 0, pr = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&pc, ols_fused_kernel<GID, false>,
                                                     FusedCfg<GID>::WG, 0) != hipSuccess ||
        pc < 1)
        pc = 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&pr, ols_fused_kernel<GID, true>,
                                                     FusedCfg<GID>::WG, 0) != hipSuccess ||
        pr < 1)
        pr = 1;
    return (pc < pr ? pc : pr) * cus;
}

int fused_max_groups(int logn, int device) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
        cus < 1)
        cus = 1;
    switch (logn) {
        case 3: return max_groups_t<fused_gid(3)>(cus);
        case 4: return max_groups_t<fused_gid(4)>(cus);
        case 5: return max_groups_t<fused_gid(5)>(cus);
        case 6: return max_groups_t<fused_gid(6)>(cus);
        case 7: return max_groups_t<fused_gid(7)>(cus);
        case 8: return max_groups_t<fused_gid(8)>(cus);
        case 9: return max_groups_t<fused_gid(9)>(cus);
        case 10: return max_groups_t<fused_gid(10)>(cus);
        case 11: return max_groups_t<fused_gid(11)>(cus);
        case 12: return max_groups_t<fused_gid(12)>(cus);
        case 13: return max_groups_t<fused_gid(13)>(cus);
        default: return cus;
    }
}

hipError_t launch_plan_taps(int logn, const float2 *taps, float2 *H, const float2 *tw,
                            hipStream_t stream) {
    switch (logn) {
        case 3: return launch_plan_t<fused_gid(3)>(taps, H, tw, stream);
        case 4: return launch_plan_t<fused_gid(4)>(taps, H, tw, stream);
        case 5: return launch_plan_t<fused_gid(5)>(taps, H, tw, stream);
        case 6: return launch_plan_t<fused_gid(6)>(taps, H, tw, stream);
        case 7: return launch_plan_t<fused_gid(7)>(taps, H, tw, stream);
        case 8: return launch_plan_t<fused_gid(8)>(taps, H, tw, stream);
        case 9: return launch_plan_t<fused_gid(9)>(taps, H, tw, stream);
        case 10: return launch_plan_t<fused_gid(10)>(taps, H, tw, stream);
        case 11: return launch_plan_t<fused_gid(11)>(taps, H, tw, stream);
        case 12: return launch_plan_t<fused_gid(12)>(taps, H, tw, stream);
        case 13: return launch_plan_t<fused_gid(13)>(taps, H, tw, stream);
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

int twiddle_count(int gid) { return make_geo(gid).twoff[make_geo(gid).npass]; }

void build_twiddles(int gid, float2 *out) {
    const Geo g = make_geo(gid);
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

void build_h_permutation(int gid, int64_t *perm) {
    const Geo g = make_geo(gid);
    for (int r = 0; r < g.P; ++r)
        for (int tb = 0; tb < g.TB; ++tb)
            perm[(int64_t)r * g.TB + tb] = bin_of_position(g, last_pass_position(g, tb, r));
}

}  // namespace firols
