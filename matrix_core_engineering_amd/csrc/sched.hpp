// Tile order and LDS swizzle: pure integer functions, usable on the host
// (tests link a host build of this header) and on the device.
//
// Tile order ("B200 GEMM Optimization Ladder", section E step 7: a fixed set
// of resident workgroups processes many tiles; check the tail and the tile
// order).  Workgroups are dispatched round-robin over the 8 XCDs of an
// MI355X, each XCD with its own L2.  The order below (1) renumbers workgroup
// ids so that the ids resident on one XCD are consecutive, then (2) walks
// the M x N tile grid in groups of `group_m` tile rows, column by column
// inside a group, so that the tiles one XCD holds at a time share a few A
// row-panels and B column-panels in that XCD's L2.
#pragma once

#ifdef __HIPCC__
#define MCE_HD __host__ __device__ __forceinline__
#else
#define MCE_HD inline
#endif

namespace mce {

constexpr int kNumXcd = 8;

// Workgroup id -> position in an XCD-major order.  Bijection on [0, nwg).
MCE_HD int xcd_major(int wg, int nwg)
{
    int q = nwg / kNumXcd, r = nwg % kNumXcd;
    int xcd = wg % kNumXcd, local = wg / kNumXcd;
    return xcd < r ? xcd * (q + 1) + local : r * (q + 1) + (xcd - r) * q + local;
}

// Position of workgroup `wg` in the tile walk: XCD-major (xcd != 0, the
// default) or the dispatch order itself (xcd == 0, for the tile-order study).
MCE_HD int wg_slot(int wg, int nwg, int xcd)
{
    return xcd ? xcd_major(wg, nwg) : wg;
}

// Tile rows per group of the grouped order: `requested` when positive
// (clamped to the tile rows), else the default of 8.
MCE_HD int group_rows(int tiles_m, int requested)
{
    const int g = requested > 0 ? requested : 8;
    return tiles_m < g ? tiles_m : g;
}

// Linear tile id -> (tile row, tile column), grouped by `group_m` tile rows.
// Bijection from [0, tiles_m * tiles_n) onto the tile grid.
MCE_HD void grouped_tile(int id, int tiles_m, int tiles_n, int group_m, int &tm, int &tn)
{
    int per_group = group_m * tiles_n;
    int g = id / per_group;
    int first_m = g * group_m;
    int rows = tiles_m - first_m < group_m ? tiles_m - first_m : group_m;
    int in_group = id - g * per_group;
    tm = first_m + in_group % rows;
    tn = in_group / rows;
}

// The r-th tile of workgroup `wg` in a persistent grid of `nwg` workgroups
// (r = 0, 1, ... while the result is < tiles_m * tiles_n), XCD-major unless
// xcd == 0.
MCE_HD int persistent_tile_id(int wg, int nwg, int r, int xcd = 1)
{
    return r * nwg + wg_slot(wg, nwg, xcd);
}

// XOR swizzle of the 16-byte chunk index inside one 128-byte LDS row (8
// chunks): the chunk stored at physical slot (c ^ swz(row)).  Rows r and r+1
// ... r+7 map one logical chunk to 8 distinct slots, and rows r and r+8 map
// it to slots of opposite parity, so 8 or 16 consecutive rows read at one
// logical chunk hit distinct banks ("B200 TMA Pipeline Designer", section B:
// a swizzle that does not match the matrix-core read pattern is a failure
// mode; here the reader and the writer use this one function).
MCE_HD int swz8(int row)
{
    return (row & 7) ^ ((row >> 3) & 1);
}

// XOR swizzle of 128-byte rows read by the 16x16x32 instruction: a fragment
// read takes rows base + (lane & 15) (base a multiple of 16) at logical
// chunk 4ks + (lane >> 4).  Of the two 16-lane read groups of a 32-lane half
// (the lane quads of equal parity of (lane >> 2) & 7), each holds eight even
// and eight odd rows, four at chunk c and four at chunk c ^ 1; row & 6 puts
// the first four on even slots and the other four on odd ones, so each
// parity of row covers all eight slots: the read is conflict-free.
MCE_HD int swz8h(int row)
{
    return row & 6;
}

// XOR swizzle for 64-byte LDS rows (4 chunks of 16 bytes).  Among rows
// r..r+7 (r even-aligned to 8) the rows of one parity map a logical chunk to
// 4 distinct slots, and among rows r, r+4, r+8, r+12 it maps to 4 distinct
// slots, so 8-lane and 16-lane groups of a 16-byte read at one logical chunk
// over consecutive rows hit distinct banks.
MCE_HD int swz4(int row)
{
    return ((row >> 1) ^ (row >> 2)) & 3;
}

// XOR swizzle for the 64-byte LDS rows of the register-staged kernel.
// Measured on gfx950 (bank-conflict counters on probe patterns): a 16-byte
// LDS read serves 16 lanes per cycle, and the 16 are the lane quads
// {0-3, 12-15, 20-23, 24-27} or {4-7, 8-11, 16-19, 28-31} of a 32-lane half
// (quad q = (lane >> 2) & 7 in group parity(q)).  A fragment read takes rows
// base + (lane & 31) at one logical chunk, so within a group each residue
// row % 4 (the row's 16-byte slot group) occurs in four quads, whose rows
// differ in bits 2-4; (row >> 3) & 3 is distinct over those four quads in
// both groups, which makes the read conflict-free.  Transposed writes of
// rows 8c + e then spread over four chunks as c varies.
MCE_HD int swz4q(int row)
{
    return (row >> 3) & 3;
}

// Whether a direct load follows the x-th of n matrix-core instructions when
// l <= n loads are spread evenly over them (load j after instruction
// floor(j*n/l)): four waves issuing a 1 KiB direct load per instruction
// would outrun the address unit (about one such load per 21 clocks per CU)
// and stall on a full queue with matrix-core work behind it.
MCE_HD constexpr bool loads_after(int x, int n, int l)
{
    return l > 0 && ((x + 1) * l + n - 1) / n > (x * l + n - 1) / n;
}

} // namespace mce
