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

// Position held by register r of thread tb in the layout of pass s (r =
// u * R[s] + j for virtual thread u, see above).
constexpr int layout_position(const Geo &g, int s, int tb, int r) {
    const int R = g.R[s], S = g.S[s];
    const int v = tb + g.TB * (r / R);
    return (v / S) * S * R + v % S + S * (r % R);
}

// Exchange between the layouts of two passes done inside the registers of
// a wave: register bit rb[i] of every thread is swapped with bit 4 + i of
// its lane (rb[i] < 0: that lane bit keeps its position bit).  Swapping
// register bit b with lane bit 4 (5) is one exchange of 16-lane (32-lane)
// rows between each pair of registers that differ in bit b.  `ok` is set
// only when every register of every thread of the block lands on the
// position the target layout assigns to it, and the block fills whole
// 32-lane halves or whole waves (TB = 32 or 64, lanes = tb).
struct LaneSwap {
    bool ok;
    int rb[2];
};
constexpr LaneSwap lane_swap_plan(const Geo &g, int from, int to) {
    LaneSwap ls{false, {-1, -1}};
    if (g.TB != 32 && g.TB != 64) return ls;
    for (int i = 0; i < 2; ++i) {
        const int lb = 4 + i;
        if ((1 << lb) >= g.TB) continue;
        // the position bit that lane bit lb carries in the source layout
        const int e = layout_position(g, from, 1 << lb, 0) - layout_position(g, from, 0, 0);
        for (int rb = 0; (1 << rb) < g.P; ++rb)
            if (layout_position(g, to, 0, 1 << rb) - layout_position(g, to, 0, 0) == e)
                ls.rb[i] = rb;
    }
    if (ls.rb[0] < 0 && ls.rb[1] < 0) return ls;
    if (ls.rb[0] == ls.rb[1]) return ls;
    for (int tb = 0; tb < g.TB; ++tb)
        for (int r = 0; r < g.P; ++r) {
            int sr = r, st = tb;   // where the value of (tb, r) comes from
            for (int i = 0; i < 2; ++i) {
                const int rb = ls.rb[i], lb = 4 + i;
                if (rb < 0) continue;
                const int c = (r >> rb) & 1, l = (tb >> lb) & 1;
                sr = (sr & ~(1 << rb)) | (l << rb);
                st = (st & ~(1 << lb)) | (c << lb);
            }
            if (layout_position(g, from, st, sr) != layout_position(g, to, tb, r)) return ls;
        }
    ls.ok = true;
    return ls;
}

}  // namespace firols
