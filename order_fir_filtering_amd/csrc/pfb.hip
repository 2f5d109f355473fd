// Polyphase filter-bank channelizer (the channelizer page, "GPU polyphase
// filter bank channelizer", sections 2.1 and 2.2) on the overlap-save
// library's register/LDS FFT.
//
// Channel c of output m is the stream shifted to baseband, filtered by the
// real prototype h (Nh taps) and decimated by D:
//   y_c(m) = sum_p h(p) xt(t_m - p) W^{c (t_m - p)},  W = exp(-2 pi j / K),
// t_m the time of the last sample of output m's hop.  With p = n K + k
// (the page's polyphase split, h_k(n) = h(n K + k)) and W^{-c n K} = 1:
//   y_c(m) = W^{c t_m} sum_k W^{-c k} v_k(m),
//   v_k(m) = sum_n h(n K + k) xt(t_m - n K - k),
// i.e. the branch filters of section 2.1, a K-point DFT across the
// branches (its bin -c mod K for channel c), and the baseband phase
// W^{c t_m}.  A workgroup takes tiles of TM consecutive outputs in time
// order: the tile's input span (T K + (TM - 1) D samples) sits in LDS, the
// part it shares with the previous tile moved there from the previous span
// and only the TM D new samples loaded from memory; then each
// group of K / 16 threads (one K-point transform, 16 points per thread)
// forms the K branch sums of one output from LDS with its taps held in
// registers, transforms them, reorders the bins through LDS into channel
// order, applies the baseband phase (t_m = t0 + m D + D - 1 mod K) and
// stores the row of K channels.
#include "pfb.hpp"

#include "ols_block.hpp"

namespace firpfb {

using firols::ic;
using firols::static_for;

namespace {

constexpr int kThreads = 256;
// LDS of one workgroup: the transforms' exchange areas (4352 values for
// every K), then the input span of at most win_cap(K, T) samples.  When a
// tile of one output per transform group fits 5600 samples even at D = K,
// the span is capped there so that two workgroups share a CU (80 KB of LDS
// and 256 VGPRs each): one loads its next tile while the other computes.
// Otherwise one workgroup takes the CU with a span of up to 14336.
constexpr int kWinSmall = 5600;
constexpr int kWinLarge = 14336;
__host__ __device__ constexpr int win_cap(int K, int T) {
    return T * K + (kThreads / (K / 16) - 1) * K <= kWinSmall ? kWinSmall : kWinLarge;
}
constexpr int kFill = 16;          // input loads in flight per thread while filling LDS
constexpr int kShift = 8;          // span values per thread per round of the LDS shift
// two floats as a clang vector, for the non-temporal store builtin
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int LOGK>
struct PfbGeo {
    static constexpr int gid = firols::geo_id(LOGK);
    static constexpr firols::Geo G = firols::make_geo(gid);
    static constexpr int K = G.N;
    static constexpr int TB = G.TB;                 // threads per transform
    static constexpr int FPW = kThreads / TB;       // transforms per workgroup at once
    static constexpr int FFT_LDS = FPW * G.lds_stride;
    static_assert(G.P == 16 && TB <= 64, "one transform inside one wave");
};

// Bin held by register r of thread tb after the forward passes.
template <int LOGK>
__device__ __forceinline__ int bin_of_register(int tb, int r) {
    constexpr firols::Geo G = PfbGeo<LOGK>::G;
    return firols::bin_of_position(G, firols::last_pass_position(G, tb, r));
}

template <int LOGK, int T>
__global__ __launch_bounds__(kThreads, win_cap(1 << LOGK, T) == kWinSmall ? 2 : 1)
void pfb_kernel(PfbArgs A) {
    using PG = PfbGeo<LOGK>;
    constexpr firols::Geo G = PG::G;
    constexpr int K = PG::K, TB = PG::TB;
    __shared__ float2 smem[PG::FFT_LDS + win_cap(K, T)];
    const int grp = threadIdx.x / TB;
    const int tb = threadIdx.x - grp * TB;
    float2 *fl = smem + grp * G.lds_stride;
    float2 *win = smem + PG::FFT_LDS;

    // this thread's taps: register r holds branch k = tb + TB pass0_m(r)
    float hr[T][16];
    static_for<0, T>([&](auto Nn) {
        constexpr int n = decltype(Nn)::value;
        static_for<0, 16>([&](auto Rr) {
            constexpr int r = decltype(Rr)::value;
            hr[n][r] = A.taps[n * K + tb + TB * firols::pass0_m<PG::gid>(r)];
        });
    });
    // the transform's twiddles in registers, loaded once (a table read per
    // pass would expose its latency to every output: one wave per SIMD)
    firols::TwRegs<PG::gid> tw;
    tw.load(A.tw, tb);
    const int Nm1 = A.Nh - 1;
    const int span = T * K + (A.TM - 1) * A.D;
    const int64_t tiles = (A.nout + A.TM - 1) / A.TM;

    // With one workgroup per CU (the large span), a workgroup takes one
    // contiguous range of tiles (the XCD's eighth of the tiles split among
    // its workgroups) in time order, so each tile after the first keeps the
    // span it shares with the previous one in LDS.  With two workgroups per
    // CU one loads while the other computes, and the tiles go round-robin
    // over the workgroups of an XCD (no shift, whose registers would spill).
    constexpr bool SLIDE = win_cap(K, T) == kWinLarge;
    int64_t t_lo, t_hi;
    {
        const int G = gridDim.x, w = blockIdx.x;
        if ((G & 7) == 0) {
            const int per = G >> 3;
            const int64_t chunk = (tiles + 7) >> 3;
            const int64_t xlo = (int64_t)(w & 7) * chunk;
            const int64_t xn = tiles - xlo < chunk ? (tiles - xlo > 0 ? tiles - xlo : 0) : chunk;
            t_lo = xlo + xn * (w >> 3) / per;
            t_hi = xlo + xn * ((w >> 3) + 1) / per;
        } else {
            t_lo = tiles * w / G;
            t_hi = tiles * (w + 1) / G;
        }
    }
    const int shift = A.TM * A.D;           // samples the span advances per tile
    const int keep = span - shift;          // samples two neighbouring tiles share

    for (int64_t it = 0;; ++it) {
        int64_t tile;
        if constexpr (SLIDE) {
            tile = t_lo + it;
            if (tile >= t_hi) break;
        } else {
            tile = firols::unit_of(tiles, blockIdx.x, gridDim.x, it);
            if (tile < 0) break;
        }
        const int64_t m0 = tile * A.TM;
        // input span of the tile: times (relative to x[0]) from w0 on
        const int64_t w0 = m0 * A.D + A.D - T * K;
        __syncthreads();                      // the previous tile's span is no longer read
        int first = 0;                        // span entries still to load
        if (SLIDE && it > 0 && keep > 0) {
            // the shared part moves to the front: each round reads its
            // values, waits for every thread, then writes them; a later
            // round's sources lie past every earlier round's destinations
            for (int e0 = 0; e0 < keep; e0 += kThreads * kShift) {
                float2 v[kShift];
                static_for<0, kShift>([&](auto Bb) {
                    constexpr int b = decltype(Bb)::value;
                    const int e = e0 + b * kThreads + (int)threadIdx.x;
                    v[b] = e < keep ? win[shift + e] : make_float2(0.f, 0.f);
                });
                __syncthreads();
                static_for<0, kShift>([&](auto Bb) {
                    constexpr int b = decltype(Bb)::value;
                    const int e = e0 + b * kThreads + (int)threadIdx.x;
                    if (e < keep) win[e] = v[b];
                });
            }
            first = keep;
        }
        // kFill loads per thread are requested before the first is written
        // to LDS, so their latencies overlap.  The sliding (one workgroup per
        // CU) form reads its input non-temporally: K = 1024, D = 512 ran
        // 92.4 -> 94.5 GS/s of input; the two-workgroup form keeps the
        // default policy (K = 128: 126.9 against 123.1 non-temporal)
        const bool inside = w0 + first >= 0 && w0 + span <= A.nsamples;
        for (int e0 = first + (int)threadIdx.x; e0 < span; e0 += kThreads * kFill) {
            float2 v[kFill];
            if (inside) {
                const float2 *__restrict__ xs = A.x + w0;
                static_for<0, kFill>([&](auto Bb) {
                    constexpr int b = decltype(Bb)::value;
                    const int e = e0 + b * kThreads;
                    if constexpr (SLIDE)
                        v[b] = e < span ? __builtin_bit_cast(float2, __builtin_nontemporal_load(
                                              (const f32x2 *)(xs + e)))
                                        : make_float2(0.f, 0.f);
                    else
                        v[b] = e < span ? xs[e] : make_float2(0.f, 0.f);
                });
            } else {
                static_for<0, kFill>([&](auto Bb) {
                    constexpr int b = decltype(Bb)::value;
                    const int64_t g = w0 + e0 + b * kThreads;
                    float2 u = make_float2(0.f, 0.f);
                    if (g >= 0) {
                        if (g < A.nsamples && e0 + b * kThreads < span) u = A.x[g];
                    } else if (g >= -(int64_t)Nm1) {
                        u = A.s_old[Nm1 + g];
                    }
                    v[b] = u;
                });
            }
            static_for<0, kFill>([&](auto Bb) {
                constexpr int b = decltype(Bb)::value;
                const int e = e0 + b * kThreads;
                if (e < span) win[e] = v[b];
            });
        }
        __syncthreads();

        for (int j = grp; j < A.TM; j += PG::FPW) {
            const int64_t m = m0 + j;
            // branch sums; the sample of tap n of branch k is at span index
            // j D + T K - 1 - n K - k
            const int base = j * A.D + T * K - 1 - tb;
            // two registers' T samples are requested together before they
            // are used, so 2 T reads are in flight instead of one
            float2 a[16];
            static_for<0, 8>([&](auto Qq) {
                constexpr int r0 = 2 * decltype(Qq)::value;
                float2 v[2][T];
                static_for<0, 2>([&](auto Ii) {
                    constexpr int i = decltype(Ii)::value;
                    constexpr int kk = TB * firols::pass0_m<PG::gid>(r0 + i);
                    static_for<0, T>([&](auto Nn) {
                        constexpr int n = decltype(Nn)::value;
                        v[i][n] = win[base - n * K - kk];
                    });
                });
                static_for<0, 2>([&](auto Ii) {
                    constexpr int i = decltype(Ii)::value;
                    float2 s = make_float2(0.f, 0.f);
                    static_for<0, T>([&](auto Nn) {
                        constexpr int n = decltype(Nn)::value;
                        s.x = fmaf(hr[n][r0 + i], v[i][n].x, s.x);
                        s.y = fmaf(hr[n][r0 + i], v[i][n].y, s.y);
                    });
                    a[r0 + i] = s;
                });
            });
            // the baseband phases W^{c t_m} of this thread's channels, requested
            // before the transform so their latency overlaps it
            const int tm = (int)((A.t0 + (m % K) * A.D + A.D - 1) & (K - 1));
            // slot jj of a thread is channel 2 (tb + TB (jj / 2)) + jj % 2: two
            // neighbouring channels per lane, so a group's stores cover whole
            // 128-byte lines even for small K
            float2 w[16];
            static_for<0, 16>([&](auto Jj) {
                constexpr int jj = decltype(Jj)::value;
                const int c = 2 * (tb + TB * (jj >> 1)) + (jj & 1);
                w[jj] = A.phase[(c * tm) & (K - 1)];
            });
            firols::forward_all<PG::gid>(tb, a, fl, tw);
            // bins to channel order: bin b is channel (K - b) mod K
            firols::wave_sync();
            static_for<0, 16>([&](auto Rr) {
                constexpr int r = decltype(Rr)::value;
                const int c = (K - bin_of_register<LOGK>(tb, r)) & (K - 1);
                fl[firols::lds_pad(G, c)] = a[r];
            });
            firols::wave_sync();
            if (m < A.nout) {
                float2 *yr = A.y + m * K;
                static_for<0, 8>([&](auto Qq) {
                    constexpr int q = decltype(Qq)::value;
                    const int c = 2 * (tb + TB * q);
                    const float2 v0 = fl[firols::lds_pad(G, c)];
                    const float2 v1 = fl[firols::lds_pad(G, c + 1)];
                    const float2 w0 = w[2 * q], w1 = w[2 * q + 1];
                    const f32x2 o0 = {v0.x * w0.x - v0.y * w0.y, v0.x * w0.y + v0.y * w0.x};
                    const f32x2 o1 = {v1.x * w1.x - v1.y * w1.y, v1.x * w1.y + v1.y * w1.x};
                    if (A.y16) {
                        const f32x4 o = {o0.x, o0.y, o1.x, o1.y};
                        __builtin_nontemporal_store(o, (f32x4 *)(yr + c));
                    } else {
                        __builtin_nontemporal_store(o0, (f32x2 *)(yr + c));
                        __builtin_nontemporal_store(o1, (f32x2 *)(yr + c + 1));
                    }
                });
            }
            firols::wave_sync();          // the exchange area is reused by the next output
        }
    }
}

// The last Nh - 1 samples of {s_old, x}.
__global__ void pfb_state_kernel(const float2 *__restrict__ x, int64_t n,
                                 const float2 *__restrict__ s_old, float2 *__restrict__ s_new,
                                 int Nm1) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= Nm1) return;
    const int64_t g = n - Nm1 + i;
    s_new[i] = g >= 0 ? x[g] : s_old[Nm1 + g];
}

template <int LOGK, int T>
const void *kernel_ptr() {
    return reinterpret_cast<const void *>(&pfb_kernel<LOGK, T>);
}

template <int LOGK>
hipError_t launch_k(const PfbArgs &a, int T, dim3 grid, hipStream_t s) {
    if (T == 2) hipLaunchKernelGGL((pfb_kernel<LOGK, 2>), grid, dim3(kThreads), 0, s, a);
    else if (T == 4) hipLaunchKernelGGL((pfb_kernel<LOGK, 4>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((pfb_kernel<LOGK, 8>), grid, dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <int LOGK>
const void *kernel_of(int T) {
    return T == 2 ? kernel_ptr<LOGK, 2>() : T == 4 ? kernel_ptr<LOGK, 4>() : kernel_ptr<LOGK, 8>();
}

int log2_of(int K) {
    int l = 0;
    while ((1 << l) < K) ++l;
    return l;
}

}  // namespace

int taps_per_branch(int K, int Nh) {
    const int t = (Nh + K - 1) / K;
    return t <= 2 ? 2 : t <= 4 ? 4 : t <= 8 ? 8 : 0;
}

int tile_outputs(int K, int D, int T) {
    const int fpw = kThreads / (K / 16);
    const int cap = win_cap(K, T);
    if (T * K + (fpw - 1) * D > cap) return 0;
    int tm = (cap - T * K) / D + 1;          // T K + (tm - 1) D <= cap
    tm -= tm % fpw;
    return tm > 8 * fpw ? 8 * fpw : tm;
}

int twiddle_count(int K) { return firols::twiddle_count(firols::geo_id(log2_of(K))); }

void build_twiddles(int K, float2 *out) { firols::build_twiddles(firols::geo_id(log2_of(K)), out); }

int max_groups(int K, int T, int device) {
    const int lk = log2_of(K);
    const void *f = lk == 6 ? kernel_of<6>(T) : lk == 7 ? kernel_of<7>(T) : lk == 8 ? kernel_of<8>(T)
                    : lk == 9 ? kernel_of<9>(T) : kernel_of<10>(T);
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
        cus < 1)
        cus = 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, f, kThreads, 0) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    return cus * per_cu;
}

hipError_t launch(const PfbArgs &a, int T, int max_groups, hipStream_t s) {
    const int lk = log2_of(a.K);
    if (a.nout <= 0 || a.TM <= 0 || (1 << lk) != a.K || lk < kMinLogK || lk > kMaxLogK ||
        (T != 2 && T != 4 && T != 8))
        return hipErrorInvalidConfiguration;
    const int64_t tiles = (a.nout + a.TM - 1) / a.TM;
    int64_t grid = tiles;
    if (grid > max_groups) grid = max_groups & ~7;    // persistent, multiple of 8
    if (grid <= 0) grid = tiles < max_groups ? tiles : max_groups;
    const dim3 g((unsigned)grid);
    hipError_t e = lk == 6   ? launch_k<6>(a, T, g, s)
                   : lk == 7 ? launch_k<7>(a, T, g, s)
                   : lk == 8 ? launch_k<8>(a, T, g, s)
                   : lk == 9 ? launch_k<9>(a, T, g, s)
                             : launch_k<10>(a, T, g, s);
    if (e != hipSuccess || a.Nh <= 1) return e;
    const int nm1 = a.Nh - 1;
    hipLaunchKernelGGL(pfb_state_kernel, dim3((unsigned)((nm1 + 255) / 256)), dim3(256), 0, s,
                       a.x, a.nsamples, a.s_old, a.s_new, nm1);
    return hipGetLastError();
}

}  // namespace firpfb
