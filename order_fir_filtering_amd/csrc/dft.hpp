// Register-resident small DFTs (radix 2, 4, 8, 16, 32) and complex helpers.
//
// dft<R, DIR> replaces a[0..R) by X[k] = sum_j a[j] * exp(DIR * 2 pi i j k / R),
// natural order in and out; DIR = -1 is the forward transform, +1 the
// unscaled inverse.  Radix 8 and 16 are split as R = R1 * R2 with input
// index j = R2*j1 + j2 and output index k = k1 + R1*k2:
//   X[k1 + R1 k2] = sum_j2 W_R^{j2 k1} (sum_j1 a[R2 j1 + j2] W_R1^{j1 k1}) W_R2^{j2 k2}.
// Every index is a compile-time constant, so the arrays live in VGPRs and
// all constant rotations (multiples of pi/16) fold into adds and at most
// four multiplies.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

namespace firols {

template <int I>
using ic = std::integral_constant<int, I>;

template <int B, int E, class F>
__host__ __device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(ic<B>{});
        static_for<B + 1, E>(f);
    }
}

__host__ __device__ __forceinline__ float2 cadd(float2 a, float2 b) {
    return make_float2(a.x + b.x, a.y + b.y);
}
__host__ __device__ __forceinline__ float2 csub(float2 a, float2 b) {
    return make_float2(a.x - b.x, a.y - b.y);
}
// a * w
__host__ __device__ __forceinline__ float2 cmul(float2 a, float2 w) {
    return make_float2(fmaf(a.x, w.x, -a.y * w.y), fmaf(a.x, w.y, a.y * w.x));
}
// a * conj(w)
__host__ __device__ __forceinline__ float2 cmulc(float2 a, float2 w) {
    return make_float2(fmaf(a.x, w.x, a.y * w.y), fmaf(a.y, w.x, -a.x * w.y));
}

// a * exp(i * A * pi / 8) for a compile-time A.
template <int A>
__host__ __device__ __forceinline__ float2 rot16(float2 a) {
    constexpr int e = ((A % 16) + 16) % 16;
    constexpr float C = 0.923879532511286756f;   // cos(pi/8)
    constexpr float S = 0.382683432365089772f;   // sin(pi/8)
    constexpr float Q = 0.707106781186547524f;   // cos(pi/4)
    if constexpr (e == 0) {
        return a;
    } else if constexpr (e == 4) {
        return make_float2(-a.y, a.x);
    } else if constexpr (e == 8) {
        return make_float2(-a.x, -a.y);
    } else if constexpr (e == 12) {
        return make_float2(a.y, -a.x);
    } else if constexpr (e == 2) {
        return make_float2((a.x - a.y) * Q, (a.x + a.y) * Q);
    } else if constexpr (e == 6) {
        return make_float2(-(a.x + a.y) * Q, (a.x - a.y) * Q);
    } else if constexpr (e == 10) {
        return make_float2((a.y - a.x) * Q, -(a.x + a.y) * Q);
    } else if constexpr (e == 14) {
        return make_float2((a.x + a.y) * Q, (a.y - a.x) * Q);
    } else {
        constexpr float c = e == 1 ? C : e == 3 ? S : e == 5 ? -S : e == 7 ? -C
                          : e == 9 ? -C : e == 11 ? -S : e == 13 ? S : C;
        constexpr float s = e == 1 ? S : e == 3 ? C : e == 5 ? C : e == 7 ? S
                          : e == 9 ? -S : e == 11 ? -C : e == 13 ? -C : -S;
        return make_float2(fmaf(a.x, c, -a.y * s), fmaf(a.x, s, a.y * c));
    }
}

// a * exp(i * A * pi / 16) for a compile-time A: even A reduce to rot16;
// odd A use cos/sin of the odd multiples of pi/16 (values of the first
// octant, mapped by symmetry).
template <int A>
__host__ __device__ __forceinline__ float2 rot32(float2 a) {
    constexpr int e = ((A % 32) + 32) % 32;
    if constexpr (e % 2 == 0) {
        return rot16<e / 2>(a);
    } else {
        constexpr float c1 = 0.980785280403230449f;  // cos(pi/16)
        constexpr float s1 = 0.195090322016128268f;  // sin(pi/16)
        constexpr float c3 = 0.831469612302545237f;  // cos(3pi/16)
        constexpr float s3 = 0.555570233019602225f;  // sin(3pi/16)
        // (cos, sin) of e*pi/16 for odd e from the quadrant and the octant
        constexpr int q = e / 8;           // quadrant: e*pi/16 in [q*pi/2, (q+1)*pi/2)
        constexpr int r = e % 8;           // 1, 3, 5, 7
        constexpr float cr = r == 1 ? c1 : r == 3 ? c3 : r == 5 ? s3 : s1;
        constexpr float sr = r == 1 ? s1 : r == 3 ? s3 : r == 5 ? c3 : c1;
        constexpr float c = q == 0 ? cr : q == 1 ? -sr : q == 2 ? -cr : sr;
        constexpr float s = q == 0 ? sr : q == 1 ? cr : q == 2 ? -sr : -cr;
        return make_float2(fmaf(a.x, c, -a.y * s), fmaf(a.x, s, a.y * c));
    }
}

template <int R, int DIR>
__host__ __device__ __forceinline__ void dft(float2 (&a)[R]);

template <int DIR>
__host__ __device__ __forceinline__ void dft2(float2 (&a)[2]) {
    float2 t = a[0];
    a[0] = cadd(t, a[1]);
    a[1] = csub(t, a[1]);
}

template <int DIR>
__host__ __device__ __forceinline__ void dft4(float2 (&a)[4]) {
    float2 t0 = cadd(a[0], a[2]);
    float2 t1 = csub(a[0], a[2]);
    float2 t2 = cadd(a[1], a[3]);
    float2 t3 = rot16<DIR * 4>(csub(a[1], a[3]));
    a[0] = cadd(t0, t2);
    a[2] = csub(t0, t2);
    a[1] = cadd(t1, t3);
    a[3] = csub(t1, t3);
}

template <int R1, int R2, int DIR>
__host__ __device__ __forceinline__ void dft_split(float2 (&a)[R1 * R2]) {
    constexpr int R = R1 * R2;
    float2 y[R];
    static_for<0, R2>([&](auto J2) {
        constexpr int j2 = decltype(J2)::value;
        float2 t[R1];
        static_for<0, R1>([&](auto J1) { t[decltype(J1)::value] = a[R2 * decltype(J1)::value + j2]; });
        dft<R1, DIR>(t);
        static_for<0, R1>([&](auto K1) {
            constexpr int k1 = decltype(K1)::value;
            y[R2 * k1 + j2] = rot32<DIR * j2 * k1 * (32 / R)>(t[k1]);
        });
    });
    static_for<0, R1>([&](auto K1) {
        constexpr int k1 = decltype(K1)::value;
        float2 t[R2];
        static_for<0, R2>([&](auto J2) { t[decltype(J2)::value] = y[R2 * k1 + decltype(J2)::value]; });
        dft<R2, DIR>(t);
        static_for<0, R2>([&](auto K2) { a[k1 + R1 * decltype(K2)::value] = t[decltype(K2)::value]; });
    });
}

template <int R, int DIR>
__host__ __device__ __forceinline__ void dft(float2 (&a)[R]) {
    static_assert(R == 1 || R == 2 || R == 4 || R == 8 || R == 16 || R == 32, "radix");
    if constexpr (R == 2) {
        dft2<DIR>(a);
    } else if constexpr (R == 4) {
        dft4<DIR>(a);
    } else if constexpr (R == 8) {
        dft_split<2, 4, DIR>(a);
    } else if constexpr (R == 16) {
        dft_split<4, 4, DIR>(a);
    } else if constexpr (R == 32) {
        dft_split<4, 8, DIR>(a);
    }
}

// The order in which dft<R> first needs its inputs: the first stage of
// dft_split<R1, R2> takes a[R2 j1 + j2] for j1 = 0 .. R1-1, one j2 after
// the other.  Loads issued in this order complete in this order, so the
// first butterflies can start before the last input arrives.
template <int R>
__host__ __device__ constexpr int dft_input_order(int i) {
    if constexpr (R == 8)
        return 4 * (i % 2) + i / 2;
    else if constexpr (R == 16)
        return 4 * (i % 4) + i / 4;
    else if constexpr (R == 32)
        return 8 * (i % 4) + i / 4;
    else
        return i;
}

// R-point DFT on a[OFF .. OFF+R) of a larger register array.
template <int R, int DIR, int OFF, int P>
__host__ __device__ __forceinline__ void dft_at(float2 (&a)[P]) {
    float2 t[R];
    static_for<0, R>([&](auto J) { t[decltype(J)::value] = a[OFF + decltype(J)::value]; });
    dft<R, DIR>(t);
    static_for<0, R>([&](auto J) { a[OFF + decltype(J)::value] = t[decltype(J)::value]; });
}

}  // namespace firols
