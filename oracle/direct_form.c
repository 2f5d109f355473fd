/*
 * Direct-form FIR oracle in float64.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library's product path links,
 * loads or calls this file; only the tests, the smoke check and the CPU
 * baseline of the benchmark do.  It shares no code with the HIP library.
 *
 * What it computes.  The method page ("一种基于GPU的高阶数字FIR滤波器频域并行
 * 处理实现方法", abstract and claim 1) filters a stream with an M-tap FIR
 * filter h by overlap-save: step 3 prefixes the first block of every call
 * with the state S0 (the M-1 samples that preceded the call) and step 5
 * keeps, of each N-point circular convolution, the L = N-M+1 points that
 * are free of wrap-around.  Every kept point is therefore exactly a term
 * of the linear convolution of h with the stream {S0, X}.  This file
 * writes that definition out, nothing more:
 *
 *     y[t] = sum_{m=0}^{M-1} h[m] * xt[t-m],   0 <= t < n,
 *     xt[j] = x[j]            for j >= 0,
 *     xt[j] = S0[M-1+j]       for -(M-1) <= j < 0  (S0[0] is the oldest).
 *
 * Arithmetic: inputs are complex64 and are widened exactly to double; the
 * taps are complex double (real taps have zero imaginary parts); every
 * product and sum is a plain double operation in order m = 0, 1, ..., M-1.
 * No FFT, no blocking, no reordering.
 */
#include <stddef.h>
#include <stdint.h>

/*
 * h      : M complex taps, interleaved (re, im) doubles.
 * s0     : M-1 complex64 state samples (interleaved floats), or NULL = zeros.
 * x      : n complex64 input samples (interleaved floats).
 * idx    : output indices to compute (each in [0, n)), or NULL = all n.
 * y      : output, one interleaved complex double per computed index.
 * nthreads: OpenMP threads for the loop over outputs (1 = serial).
 * Returns 0, or -1 on a bad argument (nothing written then).
 */
int oracle_fir_direct(const double *h, int64_t M, const float *s0,
                      const float *x, int64_t n, const int64_t *idx,
                      int64_t nidx, double *y, int nthreads)
{
    int64_t count = idx ? nidx : n;
    if (M < 1 || n < 0 || count < 0 || !h || (n > 0 && !x) ||
        (count > 0 && !y) || nthreads < 1)
        return -1;
    if (idx) {
        for (int64_t j = 0; j < nidx; ++j)
            if (idx[j] < 0 || idx[j] >= n)
                return -1;
    }
#pragma omp parallel for num_threads(nthreads) schedule(dynamic, 256)
    for (int64_t j = 0; j < count; ++j) {
        int64_t t = idx ? idx[j] : j;
        double acc_re = 0.0, acc_im = 0.0;
        for (int64_t m = 0; m < M; ++m) {
            int64_t src = t - m;
            double xr = 0.0, xi = 0.0;
            if (src >= 0) {
                xr = (double)x[2 * src];
                xi = (double)x[2 * src + 1];
            } else if (s0) {
                int64_t s = M - 1 + src;
                xr = (double)s0[2 * s];
                xi = (double)s0[2 * s + 1];
            }
            double hr = h[2 * m], hi = h[2 * m + 1];
            acc_re += hr * xr - hi * xi;
            acc_im += hr * xi + hi * xr;
        }
        y[2 * j] = acc_re;
        y[2 * j + 1] = acc_im;
    }
    return 0;
}
