// The 32768-point half-resident transform of one block (step 4 of the
// method page's claim 1), shared by the N = 32768 kernel and the
// sub-transforms of the N = 65536 paired and split kernels and of the
// N = 2^17 .. 2^20 multi-pass path: the geometry R0 = 32 of the
// half-resident transform in ols_halfres.hpp.
//
// The block (256 KB) does not fit the 160 KB LDS: pass 0 (radix 32, stride
// 1024) runs on all 32768 points in registers and leaves 32 independent
// 1024-point sub-transforms, which go through LDS in two halves of 16
// (16384 points, 132 KB with the pad slots); 512 threads hold 64 points
// each, two virtual threads v = tb and tb + 512 of 32 points in pass 0.
#pragma once

#include "ols_halfres.hpp"

namespace firols {

constexpr int kBigGid = geo_id(15, 6, 5);
constexpr Geo kBig = make_geo(kBigGid);
using Big = HalfRes<kBigGid>;
static_assert(kBig.TB == 512 && Big::R0 == 32 && Big::V == 2 && Big::NROWS == 5,
              "layout of the 32768-point half-resident transform");
constexpr int kHalf = Big::HALF;
constexpr int kHalfSlots = Big::HALF_SLOTS;
constexpr int kTw1 = Big::TW1;   // pass-1 twiddle table in LDS
using TwBig = TwHalfRes<kBigGid>;
// pass-0 twiddle rows of both virtual threads (see hr_load_rows)
using BigRows = float2[Big::V][Big::NROWS];

template <class TW>
__device__ __forceinline__ void load_big_rows(BigRows &r, const TW &tw) {
    hr_load_rows<kBigGid, 0>(r[0], tw);
    hr_load_rows<kBigGid, 1>(r[1], tw);
}

// Step 4 of one block, ending in the store (hr_transform): a holds the
// gathered block in the pass-0 layout and r the pass-0 twiddle rows;
// out(ic<U>, a) stores virtual thread U's 32 results once they are final
// and next(ic<U>, a) may then refill those registers.
template <class TW, class OUT, class NEXT>
__device__ __forceinline__ void big_transform(int tb, float2 (&a)[64], BigRows &r, float2 *lds,
                                              const TW &tw, __amdgpu_buffer_rsrc_t Hp,
                                              const OUT &out, const NEXT &next) {
    hr_transform<kBigGid>(tb, a, r, lds, tw, Hp, out, next);
}

}  // namespace firols
