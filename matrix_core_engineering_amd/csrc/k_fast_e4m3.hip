// MX E4M3 (OCP FP8 E4M3FN) levels 5-7: the launchers of the kernel
// templates in kernels_fast.hpp.
#include "kernels_fast.hpp"

namespace mce {

hipError_t launch_fast_e4m3(int level, const GemmArgs &p, hipStream_t s)
{
    return launch_fast_mx8<Mxfp8Op, Mxfp8Ring, Mxfp8Ring128, Mxfp8Ring128G, Mxfp8Ring128GW8>(level, p, s);
}

} // namespace mce
