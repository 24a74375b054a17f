// bf16 levels 4-7 for K-contiguous operands with 16-byte aligned rows: the
// launchers of the kernel templates in kernels_fast.hpp.
#include "kernels_fast.hpp"

namespace mce {

// 256x256 tiles when they give every CU work (the early-release ring when K
// is a whole number of 64-wide K tiles, at least two), else 128x128 tiles on
// the older ring, or 128x64 / 64x128 tiles (the short side across M or N)
// when 128x128 tiles would still leave CUs idle; level 7 the role-specialised
// kernel; level 9 the early-release ring with eight consumer waves (whole
// 64-wide K tiles only).  Levels 5 and 6 hand problems with a side of at
// most 64 to the skinny kernel (k_skinny.hip), whose 32-wide tiles keep
// every CU streaming.
template <bool PERSIST>
hipError_t launch_small_tiles(const GemmArgs &p, hipStream_t s)
{
    const long t128 = (long)((p.M + 127) / 128) * ((p.N + 127) / 128);
    if (t128 < p.ncu)
        return p.M >= p.N ? launch<Bf16Op, 128, 64, 3, PERSIST>(p, s) : launch<Bf16Op, 64, 128, 3, PERSIST>(p, s);
    return launch<Bf16Op, 128, 128, 3, PERSIST>(p, s);
}

hipError_t launch_fast_bf16(int level, const GemmArgs &p, hipStream_t s)
{
    // 256x256 tiles when they give every CU work, smaller ones otherwise;
    // the early-release ring needs two or more whole K tiles
    const bool big = big_tiles(p);
    const bool ring_ok = p.K > Bf16Ring64::BK && p.K % Bf16Ring64::BK == 0;
    switch (level) {
    case 4:
        return big ? launch<Bf16Op, 256, 256, 1, false>(p, s) : launch<Bf16Op, 128, 128, 1, false>(p, s);
    case 5:
        if (skinny_eligible(p))
            return launch_skinny_bf16(p, s);
        if (big && ring_ok)
            return launch_early_bf16<Bf16Ring64, Bf16Ring64S16, false>(p, s);
        return big ? launch<Bf16Op, 256, 256, 2, false>(p, s) : launch_small_tiles<false>(p, s);
    case 6:
        if (skinny_eligible(p))
            return launch_skinny_bf16(p, s);
        if (big && ring_ok)
            return launch_early_bf16<Bf16Ring64, Bf16Ring64S16, true>(p, s);
        return big ? launch<Bf16Op, 256, 256, 2, true>(p, s) : launch_small_tiles<true>(p, s);
    case 9:
        if (ring_ok)
            return launch_early_bf16<Bf16Ring64W8, Bf16Ring64S16W8, true>(p, s);
        return hipErrorInvalidValue;
    case 7:
        if (p.K > 3 * Bf16Ring::BK)
            return launch_pingpong<Bf16Ring, true>(p, s);
        return big ? launch<Bf16Op, 256, 256, 2, true>(p, s) : launch<Bf16Op, 128, 128, 3, true>(p, s);
    default:
        return hipErrorInvalidValue;
    }
}

} // namespace mce
