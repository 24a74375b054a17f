// LDS layout of MN-major operand tiles kept as loaded (k-rows of 256 bytes:
// 8-bit MX tiles of 256 rows, bf16 tiles of 128 rows), shared by the kernels
// and the host checks of the layout.
#pragma once
#include "sched.hpp"

namespace mce {

// XOR swizzle of the 16-byte chunks of k-row `krow`: a transpose read takes
// eight consecutive k-rows (8-aligned) at one chunk per 16-lane group, the
// groups of a 32-lane half at adjacent chunks 2c and 2c + 1; (krow & 7) << 1
// keeps the chunk's parity and spreads the eight rows over eight chunks, so
// 32 lanes touch 16 distinct chunks (all 64 banks once).
MCE_HD int mn_swz(int krow) { return (krow & 7) << 1; }

// The bf16 tiles of the register-staged kernel: a fragment is two 16-bit
// transpose reads (ds_read_b64_tr_b16), each 32-lane half reading k-rows
// k .. k + 3 (k a multiple of 4) at 64 consecutive bytes (one 16-lane group
// per 32-byte half); 4 (krow & 3) puts those four rows in four different
// 64-byte quarters of the banks, and the eight lanes of a 16-byte write
// fill eight chunks of one k-row.
MCE_HD int mn_swz16(int krow) { return 4 * (krow & 3); }

} // namespace mce
