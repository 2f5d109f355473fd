// Overlap-save for N = 65536: each block is split into two 32768-point
// sub-convolutions, and one workgroup runs both on the 32768-point
// half-resident transform (ols_big.hpp), one after the other.
//
// With Ns = N / 2, n = q + j Ns and k = k0 + 2 k' (a decimation in
// frequency by two):
//   X[k0 + 2 k'] = DFT_Ns(a_k0)[k'],  a_k0[q] = W_N^{q k0} (E[q] + (-1)^k0 E[q + Ns])
//   c_k0 = IDFT_Ns(X_k0 * H_k0),      H_k0[k'] = H[k0 + 2 k']
//   y[q + j Ns] = c_0[q] + (-1)^j W_N^{-q} c_1[q]
// (method page, claim 1: gather E_i with the carried state in front,
// step 3; FFT, product with H and inverse FFT, step 4; the first M-1
// points dropped, step 5).  Per block the workgroup gathers E once, keeps
// a_0 in registers and parks a_1 in its own slot of a scratch buffer;
// transforms a_0 and parks c_0 in the slot while it takes a_1 back;
// transforms a_1 and combines, y = c_0 +- W_N^{-q} c_1, straight into the
// output.  The slot (2 Ns values per workgroup) is rewritten every block,
// so it stays in the caches.
#include <cmath>
#include <vector>

#include "ols_big.hpp"

namespace firols {

namespace {

constexpr int kNs = kBig.N;        // points of a sub-transform
constexpr int kRT = 2;             // sub-transforms per block

// a_0 of one block into the pass-0 layout (register r <-> q = tb + TB m)
// and a_1 into the slot, reading E[q] and E[q + Ns] through load(j, TB m);
// W_N^q = W_N^tb W_N^{TB m}, the second factor from the LDS table wm (the
// paired kernel forms it the same way, so both compute identical values).
// E[q] of all points is requested first; E[q + Ns] goes in groups of 8
// points, the next group requested before the current one is used, so the
// registers in flight stay bounded.
template <class LOAD>
__device__ __forceinline__ void split_gather(float2 (&a)[64], int tb, const LOAD &load,
                                             float2 wt, const float2 *wm,
                                             __amdgpu_buffer_rsrc_t rslot) {
    static_for<0, 64>([&](auto Rr) {
        constexpr int r = decltype(Rr)::value;
        a[r] = load(0, kBig.TB * pass0_m<kBigGid>(r));
    });
    constexpr int G = 8;
    float2 e[2][G];
    auto issue = [&](auto Gx) {
        constexpr int g = decltype(Gx)::value;
        static_for<0, G>([&](auto Ii) {
            constexpr int i = decltype(Ii)::value;
            constexpr int off = kBig.TB * pass0_m<kBigGid>(g * G + i);
            e[g & 1][i] = load(1, off);
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
            const float2 d = csub(a[r], e[g & 1][i]);
            a[r] = cadd(a[r], e[g & 1][i]);
            buf_store_cached(cmul(d, cmul(wt, wm[pass0_m<kBigGid>(r)])), rslot,
                             (uint32_t)tb * 8u, (uint32_t)(kBig.TB * pass0_m<kBigGid>(r)) * 8u);
        });
    });
    __builtin_amdgcn_sched_barrier(0);
}

// The combine of virtual thread U: y[q] = c_0[q] + W_N^{-q} c_1[q] and
// y[q + Ns] = c_0[q] - W_N^{-q} c_1[q] for its 32 registers (c_1 in v),
// c_0 read back from the slot; in groups of 8 points like the gather.  The
// output descriptor covers the block's valid outputs only, so dropped and
// past-the-end positions fall outside it.
template <int U, bool REAL>
__device__ __forceinline__ void split_combine(const float2 (&v)[64], int tb, int qo,
                                              __amdgpu_buffer_rsrc_t rc0, float2 wt,
                                              const float2 *wm, __amdgpu_buffer_rsrc_t ry,
                                              __amdgpu_buffer_rsrc_t ry1,
                                              __amdgpu_buffer_rsrc_t ry2) {
    constexpr int G = 8;
    float2 c0[2][G];
    auto issue = [&](auto Gx) {
        constexpr int g = decltype(Gx)::value;
        static_for<0, G>([&](auto Ii) {
            constexpr int i = decltype(Ii)::value;
            constexpr int off = kBig.TB * pass0_m<kBigGid>(32 * U + g * G + i);
            c0[g & 1][i] = buf_load_cached(rc0, (uint32_t)tb * 8u, (uint32_t)off * 8u);
        });
    };
    issue(ic<0>{});
    static_for<0, 32 / G>([&](auto Gx) {
        constexpr int g = decltype(Gx)::value;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (g + 1 < 32 / G) issue(ic<g + 1>{});
        __builtin_amdgcn_sched_barrier(0);
        static_for<0, G>([&](auto Ii) {
            constexpr int i = decltype(Ii)::value;
            constexpr int r = 32 * U + g * G + i;
            constexpr int off = kBig.TB * pass0_m<kBigGid>(r);
            const float2 b1 = cmulc(v[r], cmul(wt, wm[pass0_m<kBigGid>(r)]));
            const float2 y0 = cadd(c0[g & 1][i], b1), y1 = csub(c0[g & 1][i], b1);
            if constexpr (REAL) {
                buf_store_f32(y0.x, ry1, buf_off<4>(qo + off));
                buf_store_f32(y0.y, ry2, buf_off<4>(qo + off));
                buf_store_f32(y1.x, ry1, buf_off<4>(qo + off + kNs));
                buf_store_f32(y1.y, ry2, buf_off<4>(qo + off + kNs));
            } else {
                buf_store(y0, ry, buf_off<8>(qo + off));
                buf_store(y1, ry, buf_off<8>(qo + off + kNs));
            }
        });
    });
    __builtin_amdgcn_sched_barrier(0);
}

// Channel c of real-pair input as complex samples: rows 2c and 2c + 1 of a
// float32 [2 nchan][stride] array are its real and imaginary parts.
struct RealRows {
    const float *__restrict__ x1;
    const float *__restrict__ x2;
    __device__ __forceinline__ float2 operator[](int64_t g) const {
        return make_float2(x1[g], x2[g]);
    }
};

__device__ __forceinline__ float buf_load_f32_cached(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                     uint32_t soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

}  // namespace

// REAL: the channels are pairs of real float32 rows (RealRows), read with
// two 4-byte loads per point and stored as two float rows.
template <bool REAL>
__global__ __launch_bounds__(kBig.TB) void ols_split_kernel(SplitArgs A) {
    __shared__ float2 lds[kHalfSlots + kTw1];
    __shared__ float2 wm[64];
    float2 *lds_tw = lds + kHalfSlots;
    const int tb = threadIdx.x;
    for (int e = tb; e < kTw1; e += kBig.TB) lds_tw[e] = A.tw[kBig.twoff[1] + e];
    // W_N^q = W_N^tb W_N^{TB m} for the points q = tb + TB m of a thread
    if (tb < 64) wm[tb] = A.tw_top[kNs + kBig.TB * tb];
    const float2 wt0 = A.tw_top[kNs + tb];
    // (the first barrier of the transform orders these writes before use)
    // this workgroup's slot: a_1, then c_0 (a thread reads back only the
    // positions it wrote)
    float2 *slot = A.scratch + (int64_t)blockIdx.x * (kRT * kNs);
    const __amdgpu_buffer_rsrc_t ra1 = buf_rsrc(slot, (uint32_t)kNs * 8u);
    const __amdgpu_buffer_rsrc_t rc0 = buf_rsrc(slot + kNs, (uint32_t)kNs * 8u);
    const int Mm1 = A.M - 1;
    const int64_t per_chan = A.nblk - A.blk0;    // blocks of each channel this launch runs
    const int64_t units = per_chan * A.nchan;
    // pass-0 twiddle rows of both virtual threads, the same for every block
    BigRows r;
    {
        const TwBig tw0{buf_rsrc(A.tw, (uint32_t)kBig.twoff[kBig.npass] * 8u), lds_tw, tb};
        load_big_rows(r, tw0);
    }
    for (int64_t it = 0;; ++it) {
        const int64_t gb = unit_of(units, blockIdx.x, gridDim.x, it);
        if (gb < 0) break;
        const int64_t c = gb / per_chan;
        const int64_t i = A.blk0 + (gb - c * per_chan);
        const float2 *__restrict__ xc = A.x + c * A.stride;
        const float2 *__restrict__ sc = A.s0_old + c * Mm1;
        const int64_t g0 = i * A.L - Mm1;
        // table pointers re-derived per block so their loads stay in the loop
        const float2 *twp = A.tw, *hp = A.H;
        asm volatile("" : "+s"(twp), "+s"(hp));
        const __amdgpu_buffer_rsrc_t rtw = buf_rsrc(twp, (uint32_t)kBig.twoff[kBig.npass] * 8u);
        const __amdgpu_buffer_rsrc_t rh0 = buf_rsrc(hp, (uint32_t)kNs * 8u);
        const __amdgpu_buffer_rsrc_t rh1 = buf_rsrc(hp + kNs, (uint32_t)kNs * 8u);
        const TwBig tw{rtw, lds_tw, tb};
        // (the empty asm keeps the 64 twiddle products, which do not depend
        // on the block, from being hoisted out of the loop)
        float2 wt = wt0;
        asm volatile("" : "+v"(wt.x), "+v"(wt.y));

        const float *x1 = (const float *)A.x + 2 * c * A.stride;
        const float *x2 = x1 + A.stride;
        float2 a[64];
        if (g0 >= 0 && g0 + kRT * kNs <= A.nsamples) {
            if constexpr (REAL) {
                const __amdgpu_buffer_rsrc_t rx1 = buf_rsrc(x1 + g0, (uint32_t)(kRT * kNs) * 4u);
                const __amdgpu_buffer_rsrc_t rx2 = buf_rsrc(x2 + g0, (uint32_t)(kRT * kNs) * 4u);
                split_gather(a, tb, [&](int j, int off) {
                    const uint32_t o = (uint32_t)(off + j * kNs) * 4u;
                    return make_float2(buf_load_f32_cached(rx1, (uint32_t)tb * 4u, o),
                                       buf_load_f32_cached(rx2, (uint32_t)tb * 4u, o));
                }, wt, wm, ra1);
            } else {
                const __amdgpu_buffer_rsrc_t rx = buf_rsrc(xc + g0, (uint32_t)(kRT * kNs) * 8u);
                split_gather(a, tb, [&](int j, int off) {
                    return buf_load_cached(rx, (uint32_t)tb * 8u, (uint32_t)(off + j * kNs) * 8u);
                }, wt, wm, ra1);
            }
        } else if constexpr (REAL) {
            const int64_t xs = g0 > 0 ? g0 : 0;
            int64_t xn = A.nsamples - xs;
            xn = xn < 0 ? 0 : (xn > kRT * kNs ? kRT * kNs : xn);
            const __amdgpu_buffer_rsrc_t rx1 = buf_rsrc(x1 + xs, (uint32_t)xn * 4u);
            const __amdgpu_buffer_rsrc_t rx2 = buf_rsrc(x2 + xs, (uint32_t)xn * 4u);
            const __amdgpu_buffer_rsrc_t rs = buf_rsrc(sc, g0 < 0 ? (uint32_t)Mm1 * 8u : 0u);
            const int dx = (int)(g0 - xs) + tb;
            const uint32_t ds = (uint32_t)(g0 + Mm1 + tb);   // wraps past the state (empty descriptor)
            split_gather(a, tb, [&](int j, int off) {
                const int q = off + j * kNs;
                const float2 v = buf_load_cached(rs, ((uint32_t)q + ds) * 8u, 0);
                return make_float2(buf_load_f32_cached(rx1, buf_off<4>(q + dx), 0) + v.x,
                                   buf_load_f32_cached(rx2, buf_off<4>(q + dx), 0) + v.y);
            }, wt, wm, ra1);
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
            // q + ds indexes the state (wraps past it: empty descriptor there)
            const uint32_t ds = (uint32_t)(g0 + Mm1 + tb);
            split_gather(a, tb, [&](int j, int off) {
                const int q = off + j * kNs;
                const float2 u = buf_load_cached(rx, buf_off<8>(q + dx), 0);
                const float2 v = buf_load_cached(rs, ((uint32_t)q + ds) * 8u, 0);
                return make_float2(u.x + v.x, u.y + v.y);
            }, wt, wm, ra1);
        }

        // first half-spectrum: c_0 to the slot, a_1 back from it
        big_transform(
            tb, a, r, lds, tw, rh0,
            [&](auto Uu, const float2(&v)[64]) {
                constexpr int u = decltype(Uu)::value;
                static_for<0, 32>([&](auto J) {
                    constexpr int r = 32 * u + decltype(J)::value;
                    buf_store_cached(v[r], rc0, (uint32_t)tb * 8u,
                                     (uint32_t)(kBig.TB * pass0_m<kBigGid>(r)) * 8u);
                });
            },
            [&](auto Uu, float2(&v)[64]) {
                constexpr int u = decltype(Uu)::value;
                static_for<0, 32>([&](auto J) {
                    constexpr int r = 32 * u + decltype(J)::value;
                    v[r] = buf_load_cached(ra1, (uint32_t)tb * 8u,
                                           (uint32_t)(kBig.TB * pass0_m<kBigGid>(r)) * 8u);
                });
            });

        // second half-spectrum and the combine into y
        int64_t yn = A.nsamples - i * A.L;
        if (yn > A.L) yn = A.L;
        const __amdgpu_buffer_rsrc_t ry =
            buf_rsrc(A.y + c * A.stride + i * A.L, (uint32_t)yn * 8u);
        float *y1 = (float *)A.y + 2 * c * A.stride + i * A.L;
        const __amdgpu_buffer_rsrc_t ry1 = buf_rsrc(y1, (uint32_t)yn * 4u);
        const __amdgpu_buffer_rsrc_t ry2 = buf_rsrc(y1 + A.stride, (uint32_t)yn * 4u);
        const int qo = tb - Mm1;
        big_transform(
            tb, a, r, lds, tw, rh1,
            [&](auto Uu, const float2(&v)[64]) {
                split_combine<decltype(Uu)::value, REAL>(v, tb, fresh_v(qo), rc0, wt, wm, ry, ry1,
                                                         ry2);
            },
            [&](auto, float2(&)[64]) {});

        if (i == A.nblk - 1) {
            if constexpr (REAL)
                carry_state<kBigGid>(A.nsamples, Mm1, tb, RealRows{x1, x2}, sc,
                                     A.s0_new + c * Mm1);
            else
                carry_state<kBigGid>(A.nsamples, Mm1, tb, xc, sc, A.s0_new + c * Mm1);
        }
    }
}

// Frequency response for N = RT * Ns >= 65536 (claim 1, step 1: the N-point
// DFT of the zero-padded taps), in the order the split and multi-pass
// kernels read it: H[k0 Ns + i] = DFT_N(taps)[k0 + RT k'] / N, where k' is
// the bin that the Ns-point transform's digit-reversed order puts at
// position i.  Workgroup k0 (RT of them) forms the decimated sequence
//   a_k0[q] = sum_j taps[q + j Ns] W_N^{(q + j Ns) k0},  q < Ns,
// so that DFT_N(taps)[k0 + RT k'] = DFT_Ns(a_k0)[k'], with the phases in
// float64 (the exponent reduced mod N exactly) and the sum rounded to
// float32 once; then the forward half of the Ns-point transform of
// ols_big.hpp, as ols_big_plan_taps_kernel runs it for N = Ns.
__global__ __launch_bounds__(kBig.TB) void ols_split_plan_taps_kernel(
    const float2 *__restrict__ taps, float2 *__restrict__ H, const float2 *__restrict__ tw,
    int lrt) {
    __shared__ float2 lds[kHalfSlots];
    const int tb = threadIdx.x;
    const int k0 = blockIdx.x;
    const int RT = 1 << lrt;
    const int64_t N = (int64_t)kNs << lrt;
    const TwTable<kBigGid> twt{tw, tb};
    float2 a[kBig.P];
    static_for<0, kBig.P>([&](auto Rr) {
        constexpr int r = decltype(Rr)::value;
        const int q = tb + kBig.TB * pass0_m<kBigGid>(r);
        double re = 0.0, im = 0.0;
        for (int j = 0; j < RT; ++j) {
            const int64_t n = q + (int64_t)j * kNs;
            const float2 h = taps[n];
            // W_N^{n k0} = exp(-2 pi i e / N), e = n k0 mod N
            const int64_t e = (n * k0) & (N - 1);
            double sn, cs;
            sincospi(-2.0 * (double)e / (double)N, &sn, &cs);
            re += (double)h.x * cs - (double)h.y * sn;
            im += (double)h.x * sn + (double)h.y * cs;
        }
        a[r] = make_float2((float)re, (float)im);
    });
    float2 rw[5];
    hr_load_rows<kBigGid, 0>(rw, twt);
    dft_at<32, -1, 0>(a);
    hr_pass0_twiddles<kBigGid, 0, 1, 16, false>(a, rw);
    hr_put0<kBigGid, 0, 0>(tb, a, lds);
    hr_pass0_twiddles<kBigGid, 0, 16, 32, false>(a, rw);
    hr_load_rows<kBigGid, 1>(rw, twt);
    dft_at<32, -1, 32>(a);
    hr_pass0_twiddles<kBigGid, 1, 1, 16, false>(a, rw);
    hr_put0<kBigGid, 1, 0>(tb, a, lds);
    hr_pass0_twiddles<kBigGid, 1, 16, 32, false>(a, rw);
    const float scale = 1.0f / (float)N;   // exact: N is a power of two
    float2 *__restrict__ Hk = H + (int64_t)k0 * kNs;
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
            Hk[(32 * h + k) * kBig.TB + tb] = make_float2(c[k].x * scale, c[k].y * scale);
        });
    });
}

hipError_t launch_split_plan_taps(int logn, const float2 *taps_padded, float2 *H,
                                  const float2 *tw, hipStream_t stream) {
    const int lrt = logn - kBig.logn;
    if (lrt < 1 || lrt > kMaxLogN - kBig.logn) return hipErrorInvalidValue;
    hipLaunchKernelGGL(ols_split_plan_taps_kernel, dim3(1u << lrt), dim3(kBig.TB), 0, stream,
                       taps_padded, H, tw, lrt);
    return hipGetLastError();
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

int64_t split_slot_elems(int logn) { return (int64_t)kNs * split_radix(logn); }

int split_max_groups(int device) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
        cus < 1)
        cus = 1;
    int per_cu_real = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, ols_split_kernel<false>, kBig.TB,
                                                     0) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu_real, ols_split_kernel<true>,
                                                     kBig.TB, 0) == hipSuccess &&
        per_cu_real >= 1 && per_cu_real < per_cu)
        per_cu = per_cu_real;
    return cus * per_cu;
}

hipError_t launch_split(int logn, const SplitArgs &a, int max_groups, hipStream_t stream,
                        bool real) {
    const int64_t units = (a.nblk - a.blk0) * a.nchan;
    if (units <= 0 || a.blk0 < 0 || split_radix(logn) != kRT) return hipErrorInvalidConfiguration;
    // one slot per workgroup: never more workgroups than the plan has slots
    int64_t grid = units;
    if (grid > max_groups) grid = max_groups & ~7;    // persistent, multiple of 8
    if (grid <= 0) grid = units < max_groups ? units : max_groups;
    if (real)
        hipLaunchKernelGGL(ols_split_kernel<true>, dim3((unsigned)grid), dim3(kBig.TB), 0, stream,
                           a);
    else
        hipLaunchKernelGGL(ols_split_kernel<false>, dim3((unsigned)grid), dim3(kBig.TB), 0,
                           stream, a);
    return hipGetLastError();
}

}  // namespace firols
