// MX E5M2 levels 5-7: the E4M3 kernel templates of kernels_fast.hpp with the
// matrix-core instruction's format code 1 (the same bytes per element and
// the same fragment map).
#include "kernels_fast.hpp"

namespace mce {

hipError_t launch_fast_e5m2(int level, const GemmArgs &p, hipStream_t s)
{
    return launch_fast_mx8<E5m2Op, E5m2Ring, E5m2Ring128, E5m2Ring128G, E5m2Ring128GW8>(level, p, s);
}

} // namespace mce
