// Compile-time geometry of the LDS-resident overlap-save kernel.
//
// One N-point block is transformed by TB = N / P threads that each hold P
// complex points in registers (P = 16 by default, or N itself when N < 16).  The
// transform is an in-place mixed-radix decimation-in-frequency FFT with
// radices R[0..npass-1] (one smaller radix pass first when log2(N) is not a
// multiple of log2(R), then radix-R passes; R = P unless the geometry id
// asks for a smaller R).  Pass s works at stride
// S[s] = N / (R[0] * ... * R[s]):
//
//   virtual thread v in [0, N/R[s]),  K = v / S[s],  t = v % S[s]
//   positions     p_j = K * S[s] * R[s] + t + S[s] * j,   j in [0, R[s])
//   forward       R[s]-point DFT over j, then output k times W_{S R}^{t k}
//   inverse       times conj(W_{S R}^{t k}), then R[s]-point inverse DFT
//
// A thread runs V = P / R[s] virtual threads v = tb + TB * u.  After the
// last forward pass, position q holds bin digitrev(q) of the spectrum, so
// the product with H is taken in that order and the inverse passes, run in
// reverse, restore natural order.  The positions that a thread holds in
// pass 0 are tb + TB * m, m in [0, P), which makes the gather from the
// input and the store of the output coalesced across lanes.
#pragma once

namespace firols {

constexpr int kMaxPass = 8;

struct Geo {
    int logn, logp, N, P, TB, npass;
    int R[kMaxPass];
    int S[kMaxPass];
    int twoff[kMaxPass + 1];   // start of pass s's twiddles in the table
    int lds_stride;            // padded LDS slots of one block (float2)
};

// A geometry id packs log2(N) (low byte), optionally log2(P) (next byte;
// 0 selects the default P = 16, or N when N < 16) and optionally log2 of
// the pass radix (third byte; 0 selects radix P).  With a radix below P a
// thread runs P / radix virtual threads in every pass.
constexpr int geo_id(int logn, int logp = 0, int logr = 0) {
    return logn | (logp << 8) | (logr << 16);
}

constexpr Geo make_geo(int gid) {
    Geo g{};
    const int logn = gid & 0xff;
    int logp = (gid >> 8) & 0xff;
    if (logp == 0) logp = logn >= 4 ? 4 : logn;
    int logr = (gid >> 16) & 0xff;
    if (logr == 0 || logr > logp) logr = logp;
    g.logn = logn;
    g.logp = logp;
    g.N = 1 << logn;
    g.P = 1 << logp;
    g.TB = g.N / g.P;
    int np = 0;
    const int rem = logn % logr;
    if (rem) g.R[np++] = 1 << rem;
    for (int i = 0; i < logn / logr; ++i) g.R[np++] = 1 << logr;
    g.npass = np;
    int S = g.N;
    g.twoff[0] = 0;
    for (int s = 0; s < np; ++s) {
        S /= g.R[s];
        g.S[s] = S;
        g.twoff[s + 1] = g.twoff[s] + S * (g.R[s] - 1);
    }
    g.lds_stride = g.N + (g.N >> logp);
    return g;
}

// LDS slot of position p: one pad slot after every P positions keeps the
// strided accesses of the late passes off a single bank.
constexpr int lds_pad(const Geo &g, int p) { return p + (p >> g.logp); }

// Blocks per workgroup: small transforms share a 256-lane workgroup.
constexpr int blocks_per_wg(int gid) {
    int tb = make_geo(gid).TB;
    return tb >= 256 ? 1 : 256 / tb;
}

// Spectrum bin held at position q after the forward passes (mixed-radix
// digit reversal: the digit of weight S[s] is the output index of pass s).
constexpr int bin_of_position(const Geo &g, int q) {
    int k = 0, w = 1;
    for (int s = 0; s < g.npass; ++s) {
        int d = (q / g.S[s]) % g.R[s];
        k += d * w;
        w *= g.R[s];
    }
    return k;
}

// Position of register r of thread tb after the last forward pass.
constexpr int last_pass_position(const Geo &g, int tb, int r) {
    int R = g.R[g.npass - 1];
    int u = r / R, k = r % R;
    int v = tb + g.TB * u;
    return v * R + k;
}

}  // namespace firols
