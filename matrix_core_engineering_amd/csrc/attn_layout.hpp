// LDS layout of the attention kernel's K tile and its score-column order,
// shared by the kernel and the host checks of the layout.
#pragma once
#include "sched.hpp"

namespace mce {

// Attention's score columns in key order: column j = 8q + 4h + c of a
// 32-key block (the K row that lane j of the score product supplies) is key
// 16(q >> 1) + 8h + 4(q & 1) + c, so accumulators 8t .. 8t+7 of lane half h
// hold keys 16t + 8h .. 16t + 8h + 7 in order: the operand that half
// supplies for k-step t of the P V product.
MCE_HD int attn_key_of_col(int j)
{
    const int q = j >> 3, hh = (j >> 2) & 1, c = j & 3;
    return 16 * (q >> 1) + 8 * hh + 4 * (q & 1) + c;
}

// XOR swizzle of the attention K tile's 16-byte chunks (rows of 2 * dim
// bytes).  A fragment read takes rows 32b + attn_key_of_col(l % 32) at one
// logical chunk; of each 16-lane read group those rows have distinct r & 15
// (256-byte rows, one bank row each), or distinct (r >> 1) & 7 within each
// parity of r (128-byte rows, two per bank row): conflict-free either way.
MCE_HD int swz_attn_k(int row, int dim)
{
    return dim == 128 ? (row & 15) : ((row >> 1) & 7);
}

// XOR swizzle of the attention V tile's 16-byte chunks (key rows of 2 * dim
// bytes, stored as in memory).  A P V operand fragment is two transposing
// reads (ds_read_b64_tr_b16); each 16-lane group of one reads four
// consecutive key rows k .. k + 3 (k a multiple of 4) at 32 consecutive
// bytes of d, and the two groups of a half-wave the next 32 bytes.  With
// 256-byte rows (one bank row each) the four rows' 64-byte windows go to
// four different windows (chunk XOR 4 (r & 3)); with 128-byte rows (two per
// bank row) to distinct 32-byte pairs within each (chunk XOR 2 (r & 3)):
// conflict-free either way.
MCE_HD int swz_attn_v(int row, int dim)
{
    return dim == 128 ? 4 * (row & 3) : 2 * (row & 3);
}

} // namespace mce
