// LDS layout of MN-major 8-bit operand tiles (k-rows of 256 bytes), shared
// by the kernel and the host checks of the layout.
#pragma once
#include "sched.hpp"

namespace mce {

// XOR swizzle of the 16-byte chunks of k-row `krow`: a transpose read takes
// eight consecutive k-rows (8-aligned) at one chunk per 16-lane group, the
// groups of a 32-lane half at adjacent chunks 2c and 2c + 1; (krow & 7) << 1
// keeps the chunk's parity and spreads the eight rows over eight chunks, so
// 32 lanes touch 16 distinct chunks (all 64 banks once).
MCE_HD int mn_swz(int krow) { return (krow & 7) << 1; }

} // namespace mce
