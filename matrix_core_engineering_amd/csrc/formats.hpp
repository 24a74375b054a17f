// MX element formats, numbered as the block-scaled matrix-core instruction's
// format operand (cbsz / blgp); bits per element 8, 8, 6, 6, 4.  Plain
// constants, usable on the host and on the device.
#pragma once

namespace mce {

enum { MX_E4M3 = 0, MX_E5M2 = 1, MX_E2M3 = 2, MX_E3M2 = 3, MX_E2M1 = 4 };
constexpr int mx_bits(int fmt) { return fmt <= MX_E5M2 ? 8 : fmt <= MX_E3M2 ? 6 : 4; }

} // namespace mce
